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


_NO_DEST = re.compile(r"s_(cbranch|branch|waitcnt|nop|barrier|setprio|sleep|endpgm|"
                      r"setpc|swappc|cmp|bitcmp|dcache|icache|trap|sethalt)")


def _step_flags(t, flags):
    """Known values of 64-bit scalar flag registers (first register -> -1 or
    0, and 'vcc') after instruction t, for the lane-mask idiom the compiler
    uses to route uniform branches: s_mov_b64 s[a:b], -1/0, then s_and_b64 /
    s_andn2_b64 vcc, exec, s[a:b] (exec taken as non-zero)."""
    m = re.match(r"s_mov_b64 s\[(\d+):\d+\], (-1|0)$", t)
    if m:
        return {**flags, int(m.group(1)): int(m.group(2))}
    m = re.match(r"s_(and|andn2)_b64 vcc, exec, s\[(\d+):\d+\]$", t)
    if m:
        f = dict(flags)
        v = flags.get(int(m.group(2)))
        f.pop("vcc", None)
        if v is not None:
            f["vcc"] = (v != 0) if m.group(1) == "and" else (v == 0)  # True: vcc != 0
        return f
    dest = None
    if t.startswith("s_") and not _NO_DEST.match(t):
        dest = t.split()[1].rstrip(",") if len(t.split()) > 1 else None
    elif t.startswith("v_cmp") or t.startswith("v_cmpx"):
        dest = t.split()[1].rstrip(",")
    if dest is None:
        return flags
    f = dict(flags)
    if "vcc" in dest:
        f.pop("vcc", None)
    for r in list(f):
        if r != "vcc" and re.search(r"s\[%d:" % r, dest):
            f.pop(r)
    return f


def _untracked_load_touches(instrs, labels):
    """Instructions that name a register an assembly global load writes, on
    some path from the load before any s_waitcnt on vmcnt.  Branches on vcc
    whose value the flag idiom above fixes follow the one way they can go."""
    bad = []
    for k, (t, asm) in enumerate(instrs):
        m = re.match(r"global_load_dwordx4 v\[(\d+):(\d+)\]", t)
        if not (m and asm):
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        stack, seen = [(k + 1, {})], set()
        while stack:
            j, flags = stack.pop()
            while j < len(instrs):
                key = (j, tuple(sorted(flags.items(), key=str)))
                if key in seen:
                    break
                seen.add(key)
                t2 = instrs[j][0]
                if t2.startswith("s_waitcnt") and "vmcnt" in t2:
                    break
                if _regs(t2, "v") & dst and not (t2.startswith("global_load_dwordx4")
                                                   and instrs[j][1]):
                    bad.append((t, t2))
                    break
                br = re.match(r"s_(cbranch_\w+|branch) (\.LBB\d+_\d+)", t2)
                if br:
                    kind, target = br.group(1), labels[br.group(2)]
                    if kind == "branch":
                        j = target
                        continue
                    vcc = flags.get("vcc")
                    if kind in ("cbranch_vccnz", "cbranch_vccz") and vcc is not None:
                        if vcc == (kind == "cbranch_vccnz"):
                            j = target
                            continue
                    else:
                        stack.append((target, flags))
                if re.match(r"s_(setpc|swappc|endpgm)", t2):
                    break
                flags = _step_flags(t2, flags)
                j += 1
    return bad


def test_untracked_loads_waited_before_use(device_asm):
    # Q of the 128-head kernel is loaded by assembly (the compiler would wait
    # for all earlier loads, the KV prologue included, before its first use):
    # every path from such a load must reach a vmcnt wait before anything else
    # reads, writes or copies its destination registers
    funcs = _functions(device_asm)
    n = sum(1 for f, (ins, _) in funcs.items() if "mla_" in f
            for t, asm in ins if asm and t.startswith("global_load_dwordx4 v["))
    assert n > 0
    bad = {f: _untracked_load_touches(*fl) for f, fl in funcs.items() if "mla_" in f}
    bad = {f: b for f, b in bad.items() if b}
    assert not bad, bad


def test_scanner_flags_a_planted_untracked_use():
    load = ("global_load_dwordx4 v[4:7], v[0:1], off", True)
    use = ("v_mov_b32_e32 v20, v5", False)
    wait = ("s_waitcnt vmcnt(0)", False)
    assert _untracked_load_touches([load, use], {})
    assert not _untracked_load_touches([load, wait, use], {})
    branched = [load, ("s_cbranch_scc1 .LBB0_1", False), wait, ("s_endpgm", False), use]
    assert _untracked_load_touches(branched, {".LBB0_1": 4})
    # the flag idiom: s[4:5] = -1 makes vcc = exec & ~s[4:5] zero, so the
    # vccnz branch around the wait is never taken ...
    idiom = [load, ("s_mov_b64 s[4:5], -1", False), ("s_andn2_b64 vcc, exec, s[4:5]", False),
             ("s_cbranch_vccnz .LBB0_2", False), wait, use]
    assert not _untracked_load_touches(idiom, {".LBB0_2": 5})
    # ... but with s[4:5] = 0 it is, and with s[4:5] unknown it may be
    taken = [idiom[0], ("s_mov_b64 s[4:5], 0", False)] + idiom[2:]
    assert _untracked_load_touches(taken, {".LBB0_2": 5})
    unknown = [idiom[0], ("s_cselect_b64 s[4:5], -1, 0", False)] + idiom[2:]
    assert _untracked_load_touches(unknown, {".LBB0_2": 5})


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
