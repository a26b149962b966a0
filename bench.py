#!/usr/bin/env python3
"""Throughput of paged MLA decode (absorbed-MQA form) on one MI355X.

One step = one pass of the whole hot path over one batch: the decode kernel
(page gather -> LDS ring -> QK MFMA -> online softmax -> PV MFMA -> epilogue)
and the split combine, i.e. one mla_decode_run.  The schedule (mla_decode_plan,
host side) is built once per batch before the timed region, as a serving loop
reuses it for every layer of a decode step; its host time is reported
separately as plan_ms.

Primary line: the memory-bound h_q = 16 workload (batch 64, kv_len 4096,
page 64, bf16) in HBM GB/s of algorithmic bytes (every input and output once).
"secondary" holds the h_q = 128 workload in bf16 TFLOP/s.  Inputs are seeded
synthetic N(0,1) data resident in HBM; consecutive steps cycle through
separate copies of the inputs (at least `--copies`, and enough that the other
copies stream 512 MB between two reads of one), so that a step cannot reuse
what earlier ones left in the 256 MB Infinity Cache.

The K timed steps run back to back between two HIP events and nothing else:
`ms_per_step` (and `value`) is their total time / K, gaps between steps
included.  The same K steps then run again with events around each decode
kernel and each call, which give the breakdown; events between the steps
add gaps of their own, so that pass is not the step time.  Each workload
also reports `timing`: the mean, median, min and max of the per-step decode
time (HIP events around the library's kernels), of the whole call, and the
step time when the same steps replay from hipGraphs (one captured per input
copy) beside the eager one.

`roofline.achieved` divides the algorithmic bytes (or flops) of one launch by
the decode kernel's own average duration, from HIP events that the kernel's
launch takes from its own dispatch (its start and its end, the way
hipExtLaunchKernel records them; the second pass of the timed steps);
`decode_plus_merge` gives the same figures
for the whole mla_decode_run (decode kernel and, for split requests, the
merge launch), from events the bench records around each call on the same
stream.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode: HBM GB/s at h_q=16, bf16 TFLOPS at h_q=128, % of roofline"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
KERNEL_SRC = os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc", "kernels.hip")
# other workloads measured in the same run (parity cases at full size)
SECONDARY = ("compute_b64_h128_l4096_p64", "varlen_b768_h64_l1to2048_p16",
             "fp8_b64_h16_l8192_p64", "fp8_b64_h128_l8192_p64", "int8_b64_h16_l8192_p64",
             "int8_b64_h128_l8192_p64", "fp8ckv_bf16kpe_b64_h16_l8192_p64",
             "fp8ckv_bf16kpe_b64_h128_l8192_p64", "int8ckv_bf16kpe_b64_h16_l8192_p64",
             "int8ckv_bf16kpe_b64_h128_l8192_p64", "mtp_b64_h16_q2_l4096_p64",
             "mtp_b64_h128_q2_l4096_p64", "mem_b64_h16_l4096_p32", "mem_b64_h16_l4096_p16",
             "fp16_b64_h16_l4096_p64", "fp16_b64_h128_l4096_p64", "longctx_b4_h16_l32768_p64",
             "longctx_b1_h16_l131072_p64", "longctx_b16_h64_l8192_p64",
             "longctx_b4_h128_l32768_p64")
KV_NAMES = {0: "bf16", 1: "fp8_e4m3", 2: "int8", 3: "fp8_e4m3_ckv_bf16_kpe", 4: "int8_ckv_bf16_kpe",
            5: "fp16"}
# the arithmetic type of the contractions: bf16 MFMAs (8-bit codes are
# converted to bf16 exactly), fp16 MFMAs for fp16 inputs
DTYPE_NAMES = {0: "bf16", 1: "bf16", 2: "bf16", 3: "bf16", 4: "bf16", 5: "f16"}


def kernel_name(info: dict) -> str:
    """The decode kernel a plan launches (as rocprofv3 names it)."""
    w, k, q = info["kernel_heads"], info["kv_dtype"], info["qo_len"]
    if w == 16:  # <head blocks, layout, groups staged per wave, waves>
        return "mla_decode_stream_kernel<1, %d, %s>" % (k, "1, 8" if k == 2 else "2, 4")
    if w == 32:
        return "mla_decode_ring_kernel<2, 1, 2, 1, 4>"
    causal = "true" if q > 1 else "false"
    if w == 64:
        return "mla_decode_pair_kernel<%d, %s>" % (k, causal)
    return "mla_decode_wide_kernel<%d, %s>" % (k, causal)


class Hip:
    """The few HIP event calls the bench needs (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def synth_heads(name: str) -> int:
    import synth
    return synth.WORKLOADS[name]["heads"]


def kernel_sha() -> str:
    """Hash of the sources that decide what the GPU runs, without comments and
    whitespace (so that an edit of the text alone keeps measured counters valid)."""
    import re
    h = hashlib.sha256()
    for name in ("kernels.hip", "kernels.h", "api.cpp", "planner.cpp"):
        with open(os.path.join(ROOT, "mla_paged_kv_decode_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)               # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def device_inputs(inp, copies: int):
    import numpy as np
    import torch
    d = "cuda"

    t16 = torch.float16 if inp.kv_dtype == 5 else torch.bfloat16  # fp16 inputs

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(t16).to(d)

    def i32(a):
        return torch.from_numpy(a).to(d)

    def kv(a):  # bf16 bits or 8-bit codes
        return bf(a) if a.dtype == np.uint16 else torch.from_numpy(a).to(d)

    sets = []
    base = dict(q_nope=bf(inp.q_nope), q_pe=bf(inp.q_pe), ckv=kv(inp.ckv), kpe=kv(inp.kpe),
                kv_scale=None if inp.kv_scale is None else torch.from_numpy(inp.kv_scale).to(d),
                kv_indptr=i32(inp.kv_indptr), kv_indices=i32(inp.kv_indices),
                kv_last_page_len=i32(inp.kv_last_page_len))
    sets.append(base)
    for _ in range(copies - 1):
        sets.append({k: None if v is None else v.clone() for k, v in base.items()})
    return sets


def measure(name: str, steps: int, warmup: int, copies: int, hip: Hip, head_split: int = 0,
            l2_domains: int = 0, graph: bool = False) -> dict:
    import torch
    import mla_paged_kv_decode_amd as mla
    import synth

    inp = synth.make_workload(name)
    # between two reads of one copy, the other copies stream at least 512 MB
    # (twice the Infinity Cache), so no step finds its inputs cached
    copies = max(copies, 1 + -(-512_000_000 // inp.algorithmic_bytes()))
    sets = device_inputs(inp, copies)
    B, H, Q = inp.batch, inp.num_heads, inp.qo_len
    ws = torch.empty(mla.workspace_bytes(B, H, head_split=head_split, qo_len=Q), dtype=torch.uint8,
                     device="cuda")
    t0 = time.perf_counter()
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, inp.page_size, inp.kv_dtype, ws,
                    head_split=head_split, qo_len=Q, l2_domains=l2_domains)
    plan_ms = (time.perf_counter() - t0) * 1e3
    t16 = torch.float16 if inp.kv_dtype == 5 else torch.bfloat16  # fp16 inputs: fp16 output
    outs = [(torch.empty((B * Q, H, 512), dtype=t16, device="cuda"),
             torch.empty((B * Q, H), dtype=torch.float32, device="cuda")) for _ in range(copies)]

    def step(i):
        s = sets[i % copies]
        o, lse = outs[i % copies]
        plan.run(s["q_nope"], s["q_pe"], s["ckv"], s["kpe"], s["kv_scale"], s["kv_indptr"],
                 s["kv_indices"], s["kv_last_page_len"], inp.sm_scale, o, lse)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    before = [hip.event() for _ in range(steps)]  # decode kernel (library events)
    after = [hip.event() for _ in range(steps)]
    call_end = [hip.event() for _ in range(steps)]  # end of the whole call
    start, stop = hip.event(), hip.event()
    stream = torch.cuda.current_stream().cuda_stream
    # the timed steps: nothing but the steps between the two events
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    hip.lib.hipEventRecord(start, ctypes.c_void_p(stream))
    for i in range(steps):
        step(i)
    hip.lib.hipEventRecord(stop, ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = hip.elapsed_ms(start, stop)
    # the same steps again with events around each decode kernel and each call
    # (the breakdown; the events add gaps of their own, so this pass is not the
    # step time)
    for i in range(steps):
        plan.set_events(before[i], after[i])
        step(i)
        hip.lib.hipEventRecord(call_end[i], ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    plan.set_events(None, None)
    kern = sorted(hip.elapsed_ms(before[i], after[i]) for i in range(steps))
    call = sorted(hip.elapsed_ms(before[i], call_end[i]) for i in range(steps))
    graph_ms = None
    if graph:
        # the same steps replayed from hipGraphs (one per input copy, captured
        # once): what a serving loop that captures its decode step pays
        side = torch.cuda.Stream()
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(c)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        hip.lib.hipEventRecord(start, ctypes.c_void_p(stream))
        for i in range(steps):
            graphs[i % copies].replay()
        hip.lib.hipEventRecord(stop, ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        graph_ms = hip.elapsed_ms(start, stop) / steps
        del graphs
    for e in before + after + call_end + [start, stop]:
        hip.destroy(e)
    info = plan.info()
    return dict(name=name, inp=inp, bytes=inp.algorithmic_bytes(), flops=inp.flops(),
                ms_per_step=total_ms / steps, wall_ms_per_step=wall * 1e3 / steps,
                kernel_ms=sum(kern) / len(kern), kernel_ms_min=kern[0],
                kernel_ms_median=kern[len(kern) // 2], kernel_ms_max=kern[-1],
                call_ms=sum(call) / len(call), call_ms_median=call[len(call) // 2],
                graph_ms_per_step=graph_ms, plan_ms=plan_ms, plan=info, copies=copies)


def timing_report(m: dict) -> dict:
    """Per-launch decode-kernel times (library events around that kernel),
    whole-call times (decode + merge), and the step time from hipGraph replay
    beside the eager one."""
    r = {k: round(m[k], 5) for k in ("kernel_ms", "kernel_ms_median", "kernel_ms_min",
                                      "kernel_ms_max", "call_ms", "call_ms_median",
                                      "ms_per_step")}
    g = m.get("graph_ms_per_step")
    r["graph_ms_per_step"] = round(g, 5) if g is not None else None
    return r


def roofline_report(m: dict, peaks: dict):
    """(roofline, decode_plus_merge) of one measured workload.  The roofline is
    the decode kernel's (the dominant kernel, timed alone): HBM bytes for the
    memory-bound shapes (at most 64 query vectors per request), bf16 MFMA flops
    from 128 query vectors per request.  decode_plus_merge: the same figures for
    the whole call."""
    inp, info = m["inp"], m["plan"]
    mfma = inp.num_heads * inp.qo_len >= 128

    def rate(ms):
        s_ = ms * 1e-3
        return m["bytes"] / s_ / 1e9, m["flops"] / s_ / 1e12

    gbs, tfs = rate(m["kernel_ms"])
    if mfma:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(m["name"])
    roof["kernel"] = kernel_name(info)
    roof["kernel_ms"] = round(m["kernel_ms"], 5)
    roof["kernel_dtype"] = DTYPE_NAMES[inp.kv_dtype]
    cgbs, ctfs = rate(m["call_ms"])
    dpm = {"ms": round(m["call_ms"], 5), "gbs": round(cgbs, 1), "tflops": round(ctfs, 1),
           "frac": round((ctfs / MFMA_BF16_PEAK_TFS) if mfma else (cgbs / HBM_PEAK_GBS), 4)}
    if peaks:
        meas = peaks["mfma_bf16_tflops"] if mfma else peaks["stream_read_gbs"]
        roof["frac_of_measured_peak"] = round((tfs if mfma else gbs) / meas, 4)
        dpm["frac_of_measured_peak"] = round((ctfs if mfma else cgbs) / meas, 4)
    return roof, dpm


def workload_report(m: dict, peaks: dict) -> dict:
    """Throughput of one measured workload (value per eager step) with its
    roofline entry."""
    inp = m["inp"]
    mfma = inp.num_heads * inp.qo_len >= 128
    k_s = m["kernel_ms"] * 1e-3
    gbs, tfs = m["bytes"] / k_s / 1e9, m["flops"] / k_s / 1e12
    roof, dpm = roofline_report(m, peaks)
    r = {"workload": m["name"], "kv_dtype": KV_NAMES[inp.kv_dtype], "qo_len": inp.qo_len,
         "value": round((m["flops"] / 1e12 if mfma else m["bytes"] / 1e9)
                        / (m["ms_per_step"] * 1e-3), 2),
         "unit": "TFLOP/s" if mfma else "GB/s", "ms_per_step": round(m["ms_per_step"], 5),
         "kernel_ms": round(m["kernel_ms"], 5), "kernel_gbs": round(gbs, 1),
         "kernel_tflops": round(tfs, 1), "timing": timing_report(m),
         "input_copies": m["copies"], "plan": m["plan"], "roofline": roof,
         "decode_plus_merge": dpm}
    if peaks:
        r["frac_of_measured_read_peak"] = round(gbs / peaks["stream_read_gbs"], 4)
        r["frac_of_measured_mfma_peak"] = round(tfs / peaks["mfma_bf16_tflops"], 4)
    return r


def measure_append(kv_dtype: int, n: int, steps: int, warmup: int, hip: Hip) -> dict:
    """mla_cache_append of n new tokens (bf16 in, kv_dtype cache out) into a
    cache of n slots, rows in a seeded random order.  Algorithmic bytes per
    token: 1152 read, 1152 (bf16), 576 codes + 4 scale (8-bit) or 512 codes +
    128 kpe + 4 scale (644-byte record) written, and the 8-byte slot."""
    import numpy as np
    import torch
    import mla_paged_kv_decode_amd as mla
    rng = np.random.default_rng(11)
    P = 64
    pages = n // P
    new_c = torch.randn((n, 512), dtype=torch.float32, device="cuda").to(torch.bfloat16)
    new_k = torch.randn((n, 64), dtype=torch.float32, device="cuda").to(torch.bfloat16)
    slots = torch.from_numpy(rng.permutation(n).astype(np.int64)).cuda()
    if kv_dtype == mla.KV_BF16:
        ckv = torch.empty((pages, P, 512), dtype=torch.bfloat16, device="cuda")
        kpe = torch.empty((pages, P, 64), dtype=torch.bfloat16, device="cuda")
        sc = None
        wbytes = 1152
    else:
        kpe16 = kv_dtype in (mla.KV_FP8_E4M3_KPE_BF16, mla.KV_INT8_KPE_BF16)
        ckv = torch.empty((pages, P, 512), dtype=torch.uint8, device="cuda")
        kpe = torch.empty((pages, P, 64), dtype=torch.bfloat16 if kpe16 else torch.uint8,
                          device="cuda")
        sc = torch.empty((pages, P), dtype=torch.float32, device="cuda")
        wbytes = 644 if kpe16 else 580
    for _ in range(warmup):
        mla.cache_append(new_c, new_k, slots, ckv, kpe, kv_dtype, sc)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    start, stop = hip.event(), hip.event()
    hip.lib.hipEventRecord(start, ctypes.c_void_p(stream))
    for _ in range(steps):
        mla.cache_append(new_c, new_k, slots, ckv, kpe, kv_dtype, sc)
    hip.lib.hipEventRecord(stop, ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(start, stop) / steps
    hip.destroy(start)
    hip.destroy(stop)
    nbytes = n * (1152 + wbytes + 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "append_%s_n%d" % (KV_NAMES[kv_dtype], n), "tokens": n,
            "value": round(gbs, 2), "unit": "GB/s", "ms_per_step": round(ms, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s: float) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    the first n (request, head) rows, doubling n until the run takes at least
    target_s seconds or covers the workload; scaled to GB/s of algorithmic bytes
    of the rows done.  Also: the whole tiny workload (batch 4, 16 heads, 256
    tokens) on one thread, median of 5 runs."""
    import numpy as np
    import oracle
    import synth
    nproc = os.cpu_count() or 1
    threads = nproc
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        threads = min(threads, int(env))
    total_rows = inp.batch * inp.num_heads * inp.qo_len
    n = min(total_rows, max(threads, 16))
    while True:
        rows = np.arange(n, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.decode(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices,
                      inp.kv_last_page_len, inp.sm_scale, inp.page_size, inp.kv_dtype,
                      inp.kv_scale, rows=rows, threads=threads, qo_len=inp.qo_len)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= total_rows:
            break
        n = min(total_rows, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
    frac = n / total_rows
    tiny = synth.make_workload("tiny_b4_h16_l256_p16")
    single = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.decode(tiny.q_nope, tiny.q_pe, tiny.ckv, tiny.kpe, tiny.kv_indptr,
                      tiny.kv_indices, tiny.kv_last_page_len, tiny.sm_scale, tiny.page_size,
                      tiny.kv_dtype, tiny.kv_scale, threads=1)
        single.append(time.perf_counter() - t0)
    single.sort()
    return {"value": round(inp.algorithmic_bytes() * frac / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "first %d of %d (request, head) rows of the same workload, fp64 C oracle, "
                      "%d threads, %.2f s" % (n, total_rows, threads, dt),
            "cpu_model": cpu_model(), "nproc": nproc,
            "single_thread_tiny_b4_h16_l256_p16_s": round(single[2], 5)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mem_b64_h16_l4096_p64")
    ap.add_argument("--secondary", default=",".join(SECONDARY),
                    help="comma-separated workloads also measured and reported under 'also' "
                         "('none' to skip)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--head-split", type=int, default=0,
                    help="head split for the measured workloads (0 = the planner's choice)")
    ap.add_argument("--l2-domains", type=int, default=0,
                    help="L2 domains for placing the rows of one request (0 = the "
                         "library default of 8 XCDs, 1 = no placement)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the cache-append measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the hipGraph replay timing of each workload")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured stream-read / MFMA peak kernels")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (a kernel of known "
                         "traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path is built and measured on a "
              "single MI355X (requests shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import mla_paged_kv_decode_amd as mla
    mla.load_library()
    hip = Hip()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peaks = {}
    if not args.no_peaks:
        peaks["stream_read_gbs"] = round(mla.peak_stream_read_gbs(4 << 30), 1)
        peaks["mfma_bf16_tflops"] = round(mla.peak_mfma_bf16_tflops(), 1)
        torch.cuda.empty_cache()

    prim = measure(args.workload, args.steps, args.warmup, args.copies, hip,
                   args.head_split if synth_heads(args.workload) >= 64 else 0, args.l2_domains,
                   graph=not args.no_graph)
    inp = prim["inp"]
    mfma = inp.num_heads * inp.qo_len >= 128
    per_step_s = prim["ms_per_step"] * 1e-3
    roof, dpm = roofline_report(prim, peaks)
    out = {
        "metric": METRIC,
        "value": round((prim["flops"] / 1e12 if mfma else prim["bytes"] / 1e9) / per_step_s, 2),
        "unit": "TFLOP/s" if mfma else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[inp.kv_dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "h_q": inp.num_heads,
                   "qo_len": inp.qo_len, "kv_len": int(inp.lengths[0]),
                   "page_size": inp.page_size, "kv_dtype": KV_NAMES[inp.kv_dtype],
                   "d_ckv": 512, "d_kpe": 64, "algorithmic_bytes": prim["bytes"],
                   "flops": prim["flops"], "input_copies": prim["copies"], "plan": prim["plan"],
                   "kernel_sha": kernel_sha()},
        "roofline": roof,
        "decode_plus_merge": dpm,
        "timing": timing_report(prim),
        "plan_ms": round(prim["plan_ms"], 4),
        "measured_peaks": peaks,
        "wall_ms_per_step": round(prim["wall_ms_per_step"], 5),
    }
    if args.secondary != "none":
        out["also"] = []
        for name in args.secondary.split(","):
            sec = measure(name, args.steps, args.warmup, args.copies, hip, args.head_split,
                          args.l2_domains, graph=not args.no_graph)
            out["also"].append(workload_report(sec, peaks))
            del sec
            torch.cuda.empty_cache()
    if not args.no_append:
        out["append"] = [measure_append(k, 262144, args.steps, args.warmup, hip)
                         for k in (0, 1, 2, 3)]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
