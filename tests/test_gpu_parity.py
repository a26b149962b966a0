"""GPU parity of the HIP decode path against the fp64 oracle.

Tolerances (stated for bf16 inputs): cosine distance of the whole flattened O
<= 1e-4, max |O - O_ref| <= 2e-2, max |LSE - LSE_ref| <= 1e-3; an empty
request must give O = 0 and LSE = -inf exactly.  Every input is seeded and
synthetic (synth.py); at full workload sizes the oracle
computes a sample of (request, head) rows one by one.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_common import ABS_TOL, COS_TOL, LSE_TOL, check, dev, gpu_run, host, ref  # noqa: E402,F401


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_decode_amd as mla
    mla.load_library()  # fail loudly if the HIP library is missing


RAGGED = [1, 15, 16, 17, 63, 100, 333, 1000, 2049]


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("page", [16, 32, 64])
def test_ragged_lengths_all_shapes(heads, page):
    inp = synth.make_inputs(RAGGED, heads, page, seed=100 + heads + page, poison=True,
                            extra_pages=5)
    print("case heads=%d page=%d" % (heads, page), flush=True)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("heads,hs", [(128, 1), (128, 2), (128, 4), (64, 1), (64, 2),
                                      (32, 2)])
def test_head_split_matches_oracle(heads, hs):
    inp = synth.make_inputs([700, 1, 4096, 65, 0, 1999], heads, 32, seed=300 + hs, poison=True,
                            extra_pages=3)
    print("case heads=%d head_split=%d" % (heads, hs), flush=True)
    o, lse = host(*gpu_run(inp, head_split=hs))
    check(o, lse, *ref(inp))
    o2, lse2 = host(*gpu_run(inp, head_split=hs, force_splits=3))
    check(o2, lse2, *ref(inp))


@pytest.mark.parametrize("heads,kvd", [(16, synth.KV_BF16), (32, synth.KV_BF16),
                                       (64, synth.KV_BF16), (64, synth.KV_FP16),
                                       (128, synth.KV_BF16), (16, synth.KV_FP8_E4M3),
                                       (16, synth.KV_INT8), (128, synth.KV_INT8)])
@pytest.mark.parametrize("splits", [0, 3])
def test_many_segments_per_workgroup(heads, kvd, splits):
    # few workgroups, so each runs a long list of segments: empty requests,
    # one- and two-tile ones, tile-aligned ends, chunks of split requests
    # (partials) and whole requests in one list (16-head int8: eight waves,
    # folded into four at the end of every segment)
    import mla_paged_kv_decode_amd as mla
    rng = np.random.default_rng(900 + heads + splits)
    lengths = [0, 1, 31, 32, 33, 64, 65, 96, 0, 17, 700, 1500, 2, 128, 129, 0, 250, 1000]
    lengths += [int(x) for x in rng.integers(1, 400, 22)]
    inp = synth.make_inputs(lengths, heads, 16, kvd, seed=77 + heads, poison=True, extra_pages=4)
    t = dev(inp)
    B, H = inp.batch, heads
    print("case heads=%d kv=%d splits=%d" % (heads, kvd, splits), flush=True)
    ws = torch.empty(mla.workspace_bytes(B, H, force_splits=splits, max_workers=7),
                     dtype=torch.uint8, device="cuda")
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, 16, kvd, ws, force_splits=splits,
                    max_workers=7)
    info = plan.info()
    _, wp = plan.segments()
    assert info["num_workers"] == 7 and int(np.diff(wp).max()) >= 6
    t16 = torch.float16 if kvd == synth.KV_FP16 else torch.bfloat16
    outs = []
    for _ in range(2):
        o = torch.empty((B, H, 512), dtype=t16, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        plan.run(t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_scale"], t["kv_indptr"],
                 t["kv_indices"], t["kv_last_page_len"], inp.sm_scale, o, lse)
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    check(*host(*outs[0]), *ref(inp))


def test_tiny_workload():
    inp = synth.make_workload("tiny_b4_h16_l256_p16")
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("heads", [16, 64, 128])
@pytest.mark.parametrize("splits", [2, 3, 7])
def test_forced_splits_match_oracle(heads, splits):
    inp = synth.make_inputs([700, 64, 1, 1500, 0, 129], heads, 16, seed=200 + splits,
                            poison=True)
    o, lse = host(*gpu_run(inp, force_splits=splits))
    check(o, lse, *ref(inp))


def test_kv_len_one_is_bit_exact_row():
    inp = synth.make_inputs([1] * 5, 16, 16, seed=7, poison=True, extra_pages=3)
    o, lse = gpu_run(inp)
    o = o.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(5):
        pg = int(inp.kv_indices[inp.kv_indptr[b]])
        for h in range(16):
            assert np.array_equal(o[b, h], inp.ckv[pg, 0]), (b, h)
    _, lse_ref = ref(inp)
    assert float(np.abs(lse.cpu().numpy() - lse_ref).max()) <= LSE_TOL


def test_zero_query_gives_mean():
    inp = synth.make_inputs([37, 300, 4096], 32, 64, seed=8, poison=True)
    inp.q_nope[:] = 0
    inp.q_pe[:] = 0
    o, lse = host(*gpu_run(inp))
    o_ref, lse_ref = ref(inp)
    check(o, lse, o_ref, lse_ref)
    assert np.allclose(lse, np.log([37, 300, 4096])[:, None], atol=1e-5)


def test_empty_requests():
    inp = synth.make_inputs([0, 50, 0, 0, 900, 0], 64, 32, seed=9, poison=True)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))
    assert np.all(np.isneginf(lse[[0, 2, 3, 5]]))


def test_reruns_are_bit_identical():
    inp = synth.make_inputs([3000, 17, 1024, 555], 128, 64, seed=10)
    t = dev(inp)
    o0, l0 = gpu_run(inp, t, force_splits=3)
    for _ in range(10):
        o1, l1 = gpu_run(inp, t, force_splits=3)
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


def test_page_permutation_is_bit_identical():
    inp = synth.make_inputs([777, 2048, 31], 16, 16, seed=11, extra_pages=7)
    o0, l0 = gpu_run(inp)
    rng = np.random.default_rng(1)
    perm = rng.permutation(inp.num_pages)
    ck = np.empty_like(inp.ckv)
    kp = np.empty_like(inp.kpe)
    ck[perm] = inp.ckv
    kp[perm] = inp.kpe
    inp.ckv, inp.kpe = ck, kp
    inp.kv_indices = perm[inp.kv_indices].astype(np.int32)
    o1, l1 = gpu_run(inp)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


@pytest.mark.parametrize("heads", [16, 64, 128])
@pytest.mark.parametrize("splits", [0, 3])
def test_requests_sharing_pages(heads, splits):
    # a shared prefix: request 1 starts with request 0's first 40 pages, request
    # 2 holds request 0's pages 10..29 inside its own, and request 3 reads the
    # same page twice; the kernels read pages through the table, so the result
    # is the oracle's on the shared table
    P = 16
    base = synth.make_inputs([1000, 1500, 900, 40], heads, P, seed=61, poison=True,
                             extra_pages=8)
    ind = base.kv_indices.copy()
    ip = base.kv_indptr
    r0 = ind[ip[0]:ip[1]]
    r1 = ind[ip[1]:ip[2]].copy()
    r1[:40] = r0[:40]
    r2 = ind[ip[2]:ip[3]].copy()
    r2[20:40] = r0[10:30]
    r3 = ind[ip[3]:ip[4]].copy()
    r3[2] = r3[0]
    inp = base
    # (the shared pages are full pages of request 0, so no poisoned slot of a
    # request's last page is inside another request's range)
    inp.kv_indices = np.concatenate([r0, r1, r2, r3]).astype(np.int32)
    print("case heads=%d splits=%d" % (heads, splits), flush=True)
    o, lse = host(*gpu_run(inp, force_splits=splits))
    check(o, lse, *ref(inp))


def test_outputs_stay_in_bounds():
    """Canaries around o, lse and after the workspace's used part stay intact."""
    import mla_paged_kv_decode_amd as mla
    inp = synth.make_inputs([500, 64, 1200], 64, 16, seed=12, poison=True)
    t = dev(inp)
    B, H = 3, 64
    pad = 4096
    obuf = torch.full((B * H * 512 + 2 * pad,), 12345, dtype=torch.int16, device="cuda")
    lbuf = torch.full((B * H + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + B * H * 512].view(torch.bfloat16).view(B, H, 512)
    lse = lbuf[pad:pad + B * H].view(B, H)
    ws = torch.empty(mla.workspace_bytes(B, H, force_splits=2), dtype=torch.uint8, device="cuda")
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, 16, workspace=ws, force_splits=2)
    plan.run(t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], None, t["kv_indptr"], t["kv_indices"],
             t["kv_last_page_len"], inp.sm_scale, o, lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 12345) and torch.all(obuf[-pad:] == 12345)
    assert torch.all(lbuf[:pad] == 7.0) and torch.all(lbuf[-pad:] == 7.0)
    check(*host(o, lse), *ref(inp))


@pytest.mark.parametrize("heads,kvd", [(16, synth.KV_BF16), (128, synth.KV_BF16),
                                       (16, synth.KV_FP8_E4M3), (128, synth.KV_INT8)])
def test_graph_replay_matches_eager(heads, kvd):
    # every width: the decode kernel and, for the split requests, the merge
    # launch after it, both in the graph
    import mla_paged_kv_decode_amd as mla
    inp = synth.make_inputs([1000, 4000, 64], heads, 64, kvd, seed=13)
    print("case heads=%d kv=%d" % (heads, kvd), flush=True)
    t = dev(inp)
    B, H = 3, heads
    ws = torch.empty(mla.workspace_bytes(B, H), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, 64, kvd, workspace=ws, stream=s)
        args = (t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_scale"], t["kv_indptr"],
                t["kv_indices"], t["kv_last_page_len"], inp.sm_scale, o, lse)
        plan.run(*args, stream=s)
    torch.cuda.synchronize()
    o_eager, l_eager = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(*args, stream=s)
    for _ in range(4):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_eager.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l_eager.view(torch.int32))
    check(*host(o, lse), *ref(inp))


@pytest.mark.parametrize("heads", [16, 64, 128])
def test_timing_events_keep_results(heads):
    # mla_decode_plan_set_events: the decode kernel's launch fills the two
    # events from its own dispatch.  A run with them is bit-identical to a run
    # without, the events bracket a positive time, and turning them off again
    # changes nothing either.
    import ctypes
    import mla_paged_kv_decode_amd as mla
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    inp = synth.make_inputs([1000, 4000, 64, 0], heads, 64, seed=17 + heads)
    print("case heads=%d" % heads, flush=True)
    t = dev(inp)
    B, H = 4, heads
    ws = torch.empty(mla.workspace_bytes(B, H), dtype=torch.uint8, device="cuda")
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, 64, inp.kv_dtype, workspace=ws)
    args = (t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_scale"], t["kv_indptr"],
            t["kv_indices"], t["kv_last_page_len"], inp.sm_scale)

    def run():
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
        plan.run(*args, o, lse)
        torch.cuda.synchronize()
        return o, lse

    o0, l0 = run()
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        plan.set_events(ev[0].value, ev[1].value)
        o1, l1 = run()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0, ms.value
        plan.set_events(0, 0)
        o2, l2 = run()
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    for o, lse in ((o1, l1), (o2, l2)):
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l0.view(torch.int32))
    check(*host(o0, l0), *ref(inp))


FULL_WORKLOADS = ["mem_b64_h16_l4096_p64", "compute_b64_h128_l4096_p64",
                  "varlen_b768_h64_l1to2048_p16", "fp8_b64_h16_l8192_p64",
                  "fp8_b64_h128_l8192_p64", "int8_b64_h16_l8192_p64", "int8_b64_h128_l8192_p64",
                  "fp8ckv_bf16kpe_b64_h16_l8192_p64", "fp8ckv_bf16kpe_b64_h128_l8192_p64",
                  "int8ckv_bf16kpe_b64_h16_l8192_p64", "int8ckv_bf16kpe_b64_h128_l8192_p64",
                  "mtp_b64_h16_q2_l4096_p64", "mtp_b64_h128_q2_l4096_p64",
                  "mem_b64_h16_l4096_p32", "mem_b64_h16_l4096_p16",
                  "fp16_b64_h16_l4096_p64", "fp16_b64_h128_l4096_p64",
                  "longctx_b4_h16_l32768_p64", "longctx_b1_h16_l131072_p64",
                  "longctx_b16_h64_l8192_p64", "longctx_b4_h128_l32768_p64"]


@pytest.mark.parametrize("name", FULL_WORKLOADS)
def test_full_workloads_every_row(name):
    # every measured workload at its full size, in the launch configuration the
    # bench times (the planner's default plan), against the oracle on every
    # (query, head) row: whole-O cosine distance, max |dO| and max |dLSE| at
    # the stated tolerance over all B x qo_len x H rows; NaN-poisoned padding
    inp = synth.make_workload(name, poison=True)
    print("workload", name, flush=True)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))


# ---- 8-bit latent caches: compared with the oracle on the dequantised values

KV8 = [synth.KV_FP8_E4M3, synth.KV_INT8, synth.KV_FP8_KPE16, synth.KV_INT8_KPE16]


@pytest.mark.parametrize("kv_dtype", KV8)
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("page", [16, 64])
def test_8bit_ragged_lengths(kv_dtype, heads, page):
    inp = synth.make_inputs(RAGGED, heads, page, kv_dtype, seed=400 + heads + page + kv_dtype,
                            poison=True, extra_pages=5)
    print("case kv_dtype=%d heads=%d page=%d" % (kv_dtype, heads, page), flush=True)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("kv_dtype", KV8)
@pytest.mark.parametrize("heads,splits", [(16, 2), (16, 7), (128, 3)])
def test_8bit_forced_splits(kv_dtype, heads, splits):
    inp = synth.make_inputs([700, 64, 1, 1500, 0, 129], heads, 16, kv_dtype,
                            seed=500 + splits + kv_dtype, poison=True)
    print("case kv_dtype=%d heads=%d splits=%d" % (kv_dtype, heads, splits), flush=True)
    o, lse = host(*gpu_run(inp, force_splits=splits))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("kv_dtype", KV8)
def test_8bit_reruns_are_bit_identical(kv_dtype):
    inp = synth.make_inputs([4096, 3000, 17, 1], 128, 64, kv_dtype, seed=600 + kv_dtype,
                            poison=True)
    t = dev(inp)
    o0, l0 = gpu_run(inp, t)
    for _ in range(3):
        o1, l1 = gpu_run(inp, t)
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))


@pytest.mark.parametrize("kv_dtype", KV8)
def test_8bit_quantisation_error_vs_bf16_source(kv_dtype):
    """Diagnostic: the 8-bit result against the oracle on the bf16 source the
    codes were made from (quantisation error, not kernel error).  Bounded
    loosely; the values are printed."""
    inp = synth.make_inputs([2048] * 4, 16, 64, kv_dtype, seed=700 + kv_dtype)
    o, lse = host(*gpu_run(inp))
    src = synth.MlaInputs(inp.batch, inp.num_heads, inp.page_size, synth.KV_BF16, inp.lengths,
                          inp.q_nope, inp.q_pe, inp.ckv_src, inp.kpe_src, None, inp.kv_indptr,
                          inp.kv_indices, inp.kv_last_page_len, inp.sm_scale)
    o_src, lse_src = ref(src)
    a, b = o.ravel(), o_src.ravel()
    cos = 1.0 - float(a @ b) / (np.linalg.norm(a) * np.linalg.norm(b))
    err = float(np.abs(a - b).max())
    print("kv_dtype=%d vs bf16 source: cosine distance %.3g, max abs %.3g, max |dLSE| %.3g"
          % (kv_dtype, cos, err, float(np.abs(lse - lse_src).max())), flush=True)
    assert cos < 1e-2 and err < 0.5


def test_8bit_row_widths():
    import mla_paged_kv_decode_amd as mla
    ip = np.array([0, 1], np.int32)
    lp = np.array([1], np.int32)
    ws = torch.empty(mla.workspace_bytes(1, 128), dtype=torch.uint8, device="cuda")
    plan = mla.Plan(ip, lp, 128, 16, synth.KV_FP8_E4M3, ws)
    assert plan.info()["head_split"] == 1 and plan.info()["kernel_heads"] == 128
    plan = mla.Plan(ip, lp, 64, 16, synth.KV_FP8_E4M3, ws)
    assert plan.info()["head_split"] == 4 and plan.info()["kernel_heads"] == 16
    with pytest.raises(mla.MlaError) as e:
        mla.Plan(ip, lp, 128, 16, synth.KV_INT8, ws, head_split=4)
    assert e.value.status == -2


@pytest.mark.parametrize("kv_dtype", KV8)
def test_8bit_128_heads_as_16_head_rows(kv_dtype):
    inp = synth.make_inputs([700, 1, 4096, 65, 0, 1999], 128, 32, kv_dtype, seed=900 + kv_dtype,
                            poison=True, extra_pages=3)
    o, lse = host(*gpu_run(inp, head_split=8))
    check(o, lse, *ref(inp))


def _jump_inputs(lengths, heads, kv_dtype, seed, factor, jumps):
    """Inputs whose running score maximum jumps part way through a request:
    the kpe rows of request b from token t on (for (b, t) in jumps) are
    multiplied by a power of two (exact in bf16) before any 8-bit
    quantisation, so the q_pe . kpe part of the scores grows by that factor
    while the values (ckv) keep their size.  The online softmax then has to
    rescale its accumulators after the first tile."""
    inp = synth.make_inputs(lengths, heads, 64, synth.KV_BF16, seed=seed)
    P = inp.page_size
    for b, t_from in jumps:
        toks = np.arange(t_from, int(inp.lengths[b]))
        pages = inp.kv_indices[inp.kv_indptr[b] + toks // P]
        rows = toks % P
        x = (inp.kpe[pages, rows].astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
        inp.kpe[pages, rows] = (x.view(np.uint32) >> 16).astype(np.uint16)
    if kv_dtype != synth.KV_BF16:
        ckv, kpe, scale = synth._quantize_tokens(inp.ckv, inp.kpe, kv_dtype)
        inp = synth.MlaInputs(inp.batch, inp.num_heads, P, kv_dtype, inp.lengths, inp.q_nope,
                              inp.q_pe, ckv, kpe, scale, inp.kv_indptr, inp.kv_indices,
                              inp.kv_last_page_len, inp.sm_scale, inp.ckv, inp.kpe)
    synth._poison(inp.ckv, inp.kpe, inp.kv_scale, kv_dtype, inp.kv_indptr, inp.kv_indices,
                  inp.kv_last_page_len, P, inp.num_pages)
    return inp


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8_E4M3, synth.KV_INT8_KPE16])
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("factor", [16, 64])
def test_score_jump_rescales(kv_dtype, heads, factor):
    inp = _jump_inputs([2000, 700, 3000], heads, kv_dtype, 800 + heads + factor, factor,
                       [(0, 1000), (2, 2500)])
    print("case kv_dtype=%d heads=%d factor=%d" % (kv_dtype, heads, factor), flush=True)
    o, lse = host(*gpu_run(inp))
    check(o, lse, *ref(inp))
    o2, lse2 = host(*gpu_run(inp, force_splits=3))
    check(o2, lse2, *ref(inp))


# ---- fp16 inputs (fp16 cache, queries and output) ---------------------------


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("page", [16, 64])
def test_fp16_ragged_lengths(heads, page):
    inp = synth.make_inputs(RAGGED, heads, page, synth.KV_FP16, seed=1100 + heads + page,
                            poison=True, extra_pages=5)
    print("case fp16 heads=%d page=%d" % (heads, page), flush=True)
    o, lse = gpu_run(inp)
    assert o.dtype == torch.float16
    check(*host(o, lse), *ref(inp))


@pytest.mark.parametrize("heads,splits", [(16, 3), (128, 2), (64, 5)])
def test_fp16_forced_splits_and_queries(heads, splits):
    inp = synth.make_inputs([700, 64, 1, 1500, 0, 129], heads, 16, synth.KV_FP16,
                            seed=1200 + splits, poison=True, qo_len=2)
    print("case fp16 heads=%d splits=%d qo_len=2" % (heads, splits), flush=True)
    o, lse = host(*gpu_run(inp, force_splits=splits))
    check(o, lse, *ref(inp))


@pytest.mark.parametrize("heads,lengths", [(16, [131072]), (64, [8192] * 16), (128, [32768] * 2)])
def test_many_chunk_merge_reruns_bit_identical(heads, lengths):
    # requests cut into 16 to 256 chunks go through the merge spread over the
    # GPU; its reductions have a fixed order
    import mla_paged_kv_decode_amd as mla
    inp = synth.make_inputs(lengths, heads, 64, seed=31)
    print("case heads=%d batch=%d L=%d" % (heads, len(lengths), lengths[0]), flush=True)
    t = dev(inp)
    o1, l1 = gpu_run(inp, t)
    o2, l2 = gpu_run(inp, t)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, heads, 64)
    info = plan.info()
    assert info["num_partials"] // info["num_split_requests"] > 4


@pytest.mark.parametrize("heads,hs,l2", [(16, 0, 1), (64, 0, 1), (128, 0, 1), (128, 2, 1),
                                         (16, 0, 0), (128, 0, 0), (128, 2, 0)])
def test_one_segment_fast_path_matches_general_path(heads, hs, l2):
    # The same chunks, run one per workgroup (the workgroup's segment is its own
    # index and its request is computed from it, so the segment record and the
    # page-table loads go out together: plan info one_seg = 1, req_div > 0) and
    # two per workgroup (segment range from worker_ptr, request from the
    # record): the partials and their merge are the same, so the results are
    # bit-identical, and both match the oracle on every row.  With l2 = 0 the
    # workgroups are dealt to the 8 L2 domains (the chunks of a request on one
    # of them), and the request follows from the segment's rank before the
    # dealing (plan info req_deal = 8).
    import mla_paged_kv_decode_amd as mla
    B = 64
    splits = 4 // max(hs, 1)  # 256 segments: one per workgroup of a 256-CU device
    inp = synth.make_inputs([1024] * B, heads, 64, seed=37 + heads + hs)
    t = dev(inp)
    res = []
    for mw in (0, 128):
        ws = torch.empty(mla.workspace_bytes(B, heads, head_split=hs), dtype=torch.uint8,
                         device="cuda")
        plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, heads, 64, inp.kv_dtype, ws,
                        force_splits=splits, max_workers=mw, head_split=hs, l2_domains=l2)
        info = plan.info()
        print("case heads=%d head_split=%d l2_domains=%d max_workers=%d workers=%d segments=%d "
              "one_seg=%d req_div=%d req_deal=%d" % (
                  heads, info["head_split"], l2, mw, info["num_workers"], info["num_segments"],
                  info["one_seg"], info["req_div"], info["req_deal"]), flush=True)
        o = torch.empty((B, heads, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, heads), dtype=torch.float32, device="cuda")
        plan.run(t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_scale"], t["kv_indptr"],
                 t["kv_indices"], t["kv_last_page_len"], inp.sm_scale, o, lse)
        torch.cuda.synchronize()
        res.append((o, lse, info))
    rows = res[0][2]["head_split"]
    assert res[0][2]["num_workers"] == res[0][2]["num_segments"] == splits * B * rows
    assert res[0][2]["one_seg"] == 1 and res[0][2]["req_div"] == splits * rows
    assert res[0][2]["req_deal"] == (8 if l2 == 0 else 0)
    assert res[1][2]["num_workers"] < res[1][2]["num_segments"] == splits * B * rows
    assert res[1][2]["one_seg"] == 0 and res[1][2]["req_div"] == 0
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1], res[1][1])
    o_ref, lse_ref = ref(inp)
    for o, lse, _ in res:
        check(*host(o, lse), o_ref, lse_ref)
