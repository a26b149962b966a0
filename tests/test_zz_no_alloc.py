"""mla_decode_run_noalloc (work list and split partials in the library's
per-GPU scratch array instead of a caller workspace) against mla_decode_run
on the same plan and inputs: two calls in a row on one GPU, the second with a
smaller batch, so that it runs over what the first left in the scratch.  The
two entry points launch the same kernels on the same work list, so their
outputs must be bit-identical; both are also checked against the fp64 oracle
(every row of the small case, sampled rows of the large one)."""
import ctypes

import numpy as np
import pytest
import torch

import mla_paged_kv_decode_amd as mla
import synth
import gpu_common as gc

def _both(inp, force_splits=0, host_only_plan=False):
    t = gc.dev(inp)
    B, H, Q = inp.batch, inp.num_heads, inp.qo_len
    ws = torch.empty(mla.workspace_bytes(B, H, force_splits=force_splits, qo_len=Q),
                     dtype=torch.uint8, device="cuda")
    plan = mla.Plan(inp.kv_indptr, inp.kv_last_page_len, H, inp.page_size, inp.kv_dtype, ws,
                    force_splits=force_splits, qo_len=Q)
    plan_na = plan if not host_only_plan else mla.Plan(
        inp.kv_indptr, inp.kv_last_page_len, H, inp.page_size, inp.kv_dtype, None,
        force_splits=force_splits, qo_len=Q)
    t16 = torch.float16 if inp.kv_dtype == synth.KV_FP16 else torch.bfloat16
    outs = []
    for fn in (plan.run, plan_na.run_noalloc):
        o = torch.full((B * Q, H, 512), float("nan"), dtype=t16, device="cuda")
        lse = torch.full((B * Q, H), float("nan"), dtype=torch.float32, device="cuda")
        fn(t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_scale"], t["kv_indptr"],
           t["kv_indices"], t["kv_last_page_len"], inp.sm_scale, o, lse)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return plan, outs


def _same_bits(x, y):
    return torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                       y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32))


@pytest.mark.gpu
def test_noalloc_matches_run_two_calls_smaller_second():
    # call 1: batch 64, 128 heads, 4096 tokens (every request cut into chunks,
    # 64 MiB of partials in the scratch)
    big = synth.make_inputs([4096] * 64, 128, 64, seed=3)
    plan, ((o1, l1), (o2, l2)) = _both(big)
    assert plan.info()["num_partials"] > 0
    assert _same_bits(o1, o2) and _same_bits(l1, l2)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(64 * 128, 64, replace=False)).astype(np.int32)
    o_ref, lse_ref = gc.ref(big, rows=rows)
    o, lse = gc.host(o2, l2)
    gc.check(o.reshape(-1, 512)[rows], lse.reshape(-1)[rows], o_ref, lse_ref)
    del big, o1, o2, l1, l2
    torch.cuda.empty_cache()

    # call 2: a smaller batch over the scratch the first call left, with a
    # host-only plan (no workspace at all) and forced splits
    small = synth.make_inputs([700, 1, 333, 64, 1000, 17, 256, 5], 16, 16, seed=4,
                              poison=True, extra_pages=3)
    plan, ((o1, l1), (o2, l2)) = _both(small, force_splits=3, host_only_plan=True)
    assert plan.info()["num_partials"] > 0
    assert _same_bits(o1, o2) and _same_bits(l1, l2)
    o_ref, lse_ref = gc.ref(small)
    gc.check(*gc.host(o2, l2), o_ref, lse_ref)


def test_noalloc_rejects_plan_beyond_scratch():
    # host-only: the size is checked before any device call
    # 64 requests x 128 heads cut into 8 chunks each: 128 MiB of partials
    ip = np.arange(0, 64 * 64 + 1, 64, dtype=np.int32)
    lp = np.full(64, 64, np.int32)
    plan = mla.Plan(ip, lp, 128, 64, mla.KV_BF16, None, num_cus=256, force_splits=8)
    lib = mla.load_library()
    st = lib.mla_decode_run_noalloc(plan._h, None, None, None, None, None, None, None, None,
                                    ctypes.c_float(0.1), None, None, None)
    assert st == -3
    assert b"scratch" in lib.mla_last_error()
