"""Helpers shared by the GPU parity tests: device copies of synthetic inputs,
one-shot runs through the C ABI, the fp64 oracle reference and the tolerance
check (cosine distance of the whole flattened O <= 1e-4, max |O - O_ref| <=
2e-2, max |LSE - LSE_ref| <= 1e-3; rows with no visible token must give O = 0
and LSE = -inf exactly)."""
import numpy as np
import torch

import oracle
import synth

COS_TOL, ABS_TOL, LSE_TOL = 1e-4, 2e-2, 1e-3


def dev(inp):
    d = "cuda"
    t = {}
    t16 = torch.float16 if inp.kv_dtype == synth.KV_FP16 else torch.bfloat16
    t["q_nope"] = torch.from_numpy(inp.q_nope.view(np.int16)).view(t16).to(d)
    t["q_pe"] = torch.from_numpy(inp.q_pe.view(np.int16)).view(t16).to(d)
    if inp.kv_dtype in (synth.KV_BF16, synth.KV_FP16):
        t["ckv"] = torch.from_numpy(inp.ckv.view(np.int16)).view(t16).to(d)
        t["kpe"] = torch.from_numpy(inp.kpe.view(np.int16)).view(t16).to(d)
        t["kv_scale"] = None
    else:
        t["ckv"] = torch.from_numpy(inp.ckv).to(d)
        if inp.kpe.dtype == np.uint16:  # bf16 kpe of the 644-byte record
            t["kpe"] = torch.from_numpy(inp.kpe.view(np.int16)).view(torch.bfloat16).to(d)
        else:
            t["kpe"] = torch.from_numpy(inp.kpe).to(d)
        t["kv_scale"] = torch.from_numpy(inp.kv_scale).to(d)
    for k in ("kv_indptr", "kv_indices", "kv_last_page_len"):
        t[k] = torch.from_numpy(getattr(inp, k)).to(d)
    return t


def gpu_run(inp, t=None, force_splits=0, head_split=0):
    import mla_paged_kv_decode_amd as mla
    t = t or dev(inp)
    o, lse = mla.decode(t["q_nope"], t["q_pe"], t["ckv"], t["kpe"], t["kv_indptr"],
                        t["kv_indices"], t["kv_last_page_len"], inp.sm_scale, inp.kv_dtype,
                        t["kv_scale"], kv_indptr_host=inp.kv_indptr,
                        kv_last_page_len_host=inp.kv_last_page_len, force_splits=force_splits,
                        head_split=head_split, qo_len=inp.qo_len)
    torch.cuda.synchronize()
    return o, lse


def host(o, lse):
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(inp, rows=None):
    return oracle.decode(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices,
                         inp.kv_last_page_len, inp.sm_scale, inp.page_size, inp.kv_dtype,
                         inp.kv_scale, rows=rows, qo_len=inp.qo_len)


def check(o, lse, o_ref, lse_ref):
    o = o.reshape(-1, 512)
    lse = lse.reshape(-1)
    o_ref = o_ref.reshape(-1, 512)
    lse_ref = lse_ref.reshape(-1)
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0)
    ne = ~empty
    if not ne.any():
        return
    a, b = o[ne].ravel(), o_ref[ne].ravel()
    assert np.all(np.isfinite(a)), "non-finite output"
    cos = 1.0 - float(a @ b) / (np.linalg.norm(a) * np.linalg.norm(b))
    err = float(np.abs(a - b).max())
    lerr = float(np.abs(lse[ne] - lse_ref[ne]).max())
    assert cos <= COS_TOL, ("cosine distance", cos)
    assert err <= ABS_TOL, ("max abs", err)
    assert lerr <= LSE_TOL, ("lse", lerr)
