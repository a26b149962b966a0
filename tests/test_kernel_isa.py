"""CPU checks of the compiled gfx950 decode kernels (device assembly from hipcc).

The 128-head kernel issues its MFMAs as inline assembly: PV with the O^T
accumulators pinned to AGPRs, QK with the scores in VGPRs.  The compiler does
not know the latency of an MFMA it did not emit, so it inserts no wait states
before a later read of those registers; a read it adds on its own (a copy of
an accumulator block between registers, which happens when the loop runs short
of registers) would then see the value from before the MFMA.  This test
compiles the kernels and fails if any instruction other than an MFMA that
names a register written by such an MFMA comes before 18 wait states have
passed (the 32x32 MFMA needs fewer; 18 leaves room), counting s_nop N as N + 1
and following every branch (the compiler places such copies and spills on the
paths that leave the loop as readily as inside it).
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
WAIT_STATES = 18


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc missing")
    tmp = tempfile.mkdtemp()
    try:
        out = os.path.join(tmp, "kernels.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", "-Wno-inline-asm",
               "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc"),
               os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc", "kernels.hip"), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        yield open(out).read()
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _functions(asm):
    """name -> (instructions, labels): instructions carry an in-asm flag, labels
    map a branch target to the index of the instruction that follows it."""
    funcs = {}
    name = None
    in_asm = False
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            funcs[name] = ([], {})
            in_asm = False
            continue
        if name is None:
            continue
        instrs, labels = funcs[name]
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        lb = re.match(r"^(\.LBB\d+_\d+):", t)
        if lb:
            labels[lb.group(1)] = len(instrs)
            continue
        if t == "s_endpgm":
            instrs.append((t, in_asm))
            name = None
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        instrs.append((t, in_asm))
    return funcs


def _regs(t, kind):
    """Registers of one file ('a' or 'v') that instruction t names."""
    regs = set()
    for m in re.finditer(r"\b%s\[(\d+):(\d+)\]" % kind, t):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\b%s(\d+)\b" % kind, t):
        regs.add(int(m.group(1)))
    return regs


def _first_touch(instrs, labels, j, kind, dst, ws, seen):
    """First non-MFMA instruction on any path from j that names a register of
    dst (file `kind`) before WAIT_STATES have passed (s_nop N counts N + 1), or
    None."""
    while j < len(instrs) and ws < WAIT_STATES:
        if (j, ws) in seen:
            return None
        seen.add((j, ws))
        t = instrs[j][0]
        if not t.startswith("v_mfma") and _regs(t, kind) & dst:
            return (t, ws)
        n = re.match(r"s_nop (\d+)", t)
        ws += int(n.group(1)) + 1 if n else 1
        br = re.match(r"s_(cbranch_\w+|branch) (\.LBB\d+_\d+)", t)
        if br:
            hit = _first_touch(instrs, labels, labels[br.group(2)], kind, dst, ws, seen)
            if hit or br.group(1) == "branch":
                return hit
        if re.match(r"s_(setpc|swappc|endpgm)", t):
            return None
        j += 1
    return None


def _early_agpr_reads(instrs, labels=None):
    labels = labels or {}
    bad = []
    for k, (t, asm) in enumerate(instrs):
        m = re.match(r"v_mfma_f32_32x32x16_\w+ ([av])\[(\d+):(\d+)\]", t)
        if not (m and asm):
            continue
        dst = set(range(int(m.group(2)), int(m.group(3)) + 1))
        hit = _first_touch(instrs, labels, k + 1, m.group(1), dst, 0, set())
        if hit:
            bad.append((t,) + hit)
    return bad


def test_compiled_kernels_present(device_asm):
    funcs = _functions(device_asm)
    wide = [f for f in funcs if "mla_decode_wide_kernel" in f]
    assert len(wide) == 12  # 6 cache layouts x causal / not
    assert any("mla_decode_stream_kernel" in f for f in funcs)


def test_no_accumulator_read_before_asm_mfma_completes(device_asm):
    funcs = _functions(device_asm)
    bad = {f: _early_agpr_reads(*fl) for f, fl in funcs.items() if "mla_" in f}
    bad = {f: b for f, b in bad.items() if b}
    assert not bad, bad


def test_scanner_flags_a_planted_early_read():
    # the check itself: an AGPR read right after an asm MFMA is found, one after
    # enough s_nop wait states is not, and a read behind a branch is followed
    early = [("v_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]", True),
             ("s_add_i32 s1, s1, 1", False), ("v_accvgpr_read_b32 v0, a16", False)]
    late = [early[0], ("s_nop 7", True), ("s_nop 7", True), ("s_nop 3", True), early[2]]
    other = [early[0], ("v_accvgpr_read_b32 v0, a32", False)]
    assert _early_agpr_reads(early) and not _early_agpr_reads(late)
    assert not _early_agpr_reads(other)
    # loop exit: the read sits behind a conditional branch, past an s_endpgm
    branched = [early[0], ("s_cbranch_scc1 .LBB0_9", False), ("s_endpgm", False),
                ("scratch_store_dword off, v0, off", False), ("v_accvgpr_read_b32 v0, a22", False)]
    assert _early_agpr_reads(branched, {".LBB0_9": 4})
    assert not _early_agpr_reads(branched[:3], {".LBB0_9": 3})
    # a write of the accumulator (zeroing it for the next segment) counts too
    zero = [early[0], ("s_branch .LBB0_2", False), ("s_endpgm", False),
            ("v_accvgpr_write_b32 a31, 0", False)]
    assert _early_agpr_reads(zero, {".LBB0_2": 3})
    # an accumulator in VGPRs: a VALU read of the scores too soon is found, one
    # of another register is not
    vform = [("v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[4:7], v[32:47]", True),
             ("v_max_f32_e32 v48, v40, v48", False)]
    assert _early_agpr_reads(vform)
    assert not _early_agpr_reads([vform[0], ("v_max_f32_e32 v48, v30, v48", False)])
