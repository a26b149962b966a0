"""A plan made at one set of lengths, reused while every request grows.

mla_decode_plan fixes the chunk boundaries it cuts, but the last chunk of
every request ends at the request's length as the device page table gives it
at run time, so a decode loop can keep one plan (and one captured graph) while
it appends tokens.  Here the plan and a hipGraph of mla_decode_run are made at
lengths L (one request empty); then, for g = 1 .. 16, every request gains g
tokens (new slots in its last page, or a new page), the device page table is
rewritten in place, and the graph is replayed: each replay must be
bit-identical to an eager run of the same plan and match the fp64 oracle at
lengths L + g within the stated tolerance.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_common import check, host, ref  # noqa: E402

P = 16
L0 = [1000, 4096, 77, 0, 2048, 31]
GROW = 16


def _tables(pages_of, lengths):
    """CSR page table of requests with `lengths` tokens, each using the first
    pages of its own page list."""
    n = [(L + P - 1) // P for L in lengths]
    indptr = np.zeros(len(lengths) + 1, np.int32)
    indptr[1:] = np.cumsum(n)
    indices = np.concatenate([pages_of[b][:n[b]] for b in range(len(lengths))]).astype(np.int32)
    last = np.array([L - (k - 1) * P if k > 0 else 1 for L, k in zip(lengths, n)], np.int32)
    return indptr, indices, last


@pytest.mark.parametrize("heads,kvd,splits,q", [(16, synth.KV_BF16, 0, 1),
                                                (16, synth.KV_FP8_E4M3, 3, 1),
                                                (64, synth.KV_BF16, 0, 1),
                                                (128, synth.KV_BF16, 4, 1),
                                                (16, synth.KV_BF16, 2, 4)])
def test_plan_and_graph_survive_growth(heads, kvd, splits, q):
    import mla_paged_kv_decode_amd as mla
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load_library()
    # cache and page lists sized for the grown lengths
    full = synth.make_inputs([L + GROW for L in L0], heads, P, kvd, seed=71 + heads, poison=True,
                             extra_pages=4, qo_len=q)
    pages_of = [full.kv_indices[full.kv_indptr[b]:full.kv_indptr[b + 1]] for b in range(len(L0))]
    B, H = len(L0), heads
    d = "cuda"
    t16 = torch.bfloat16
    qn = torch.from_numpy(full.q_nope.view(np.int16)).view(t16).to(d)
    qp = torch.from_numpy(full.q_pe.view(np.int16)).view(t16).to(d)
    if kvd == synth.KV_BF16:
        ckv = torch.from_numpy(full.ckv.view(np.int16)).view(t16).to(d)
        kpe = torch.from_numpy(full.kpe.view(np.int16)).view(t16).to(d)
        sc = None
    else:
        ckv = torch.from_numpy(full.ckv).to(d)
        kpe = torch.from_numpy(full.kpe).to(d)
        sc = torch.from_numpy(full.kv_scale).to(d)
    cap = int(full.kv_indptr[-1])
    ip_d = torch.zeros(B + 1, dtype=torch.int32, device=d)
    ix_d = torch.zeros(cap, dtype=torch.int32, device=d)
    lp_d = torch.zeros(B, dtype=torch.int32, device=d)

    def upload(lengths):
        ip, ix, lp = _tables(pages_of, lengths)
        ip_d.copy_(torch.from_numpy(ip))
        ix_d[:ix.size].copy_(torch.from_numpy(ix))
        lp_d.copy_(torch.from_numpy(lp))
        torch.cuda.synchronize()
        return ip, ix, lp

    ip0, _, lp0 = upload(L0)
    ws = torch.empty(mla.workspace_bytes(B, H, force_splits=splits, qo_len=q), dtype=torch.uint8,
                     device=d)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        plan = mla.Plan(ip0, lp0, H, P, kvd, ws, force_splits=splits, stream=side, qo_len=q)
    side.synchronize()
    print("case heads=%d kv=%d splits=%d qo_len=%d plan %s" % (heads, kvd, splits, q, plan.info()),
          flush=True)
    o_g = torch.empty((B * q, H, 512), dtype=t16, device=d)
    l_g = torch.empty((B * q, H), dtype=torch.float32, device=d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run(qn, qp, ckv, kpe, sc, ip_d, ix_d, lp_d, full.sm_scale, o_g, l_g, stream=side)
    for grow in range(1, GROW + 1):
        lengths = [L + grow for L in L0]
        ip, ix, lp = upload(lengths)
        g.replay()
        torch.cuda.synchronize()
        o_e = torch.empty_like(o_g)
        l_e = torch.empty_like(l_g)
        plan.run(qn, qp, ckv, kpe, sc, ip_d, ix_d, lp_d, full.sm_scale, o_e, l_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), grow
        assert torch.equal(l_g, l_e), grow
        cur = synth.MlaInputs(B, H, P, kvd, np.asarray(lengths, np.int64), full.q_nope,
                              full.q_pe, full.ckv, full.kpe, full.kv_scale, ip, ix, lp,
                              full.sm_scale, qo_len=q)
        check(*host(o_g, l_g), *ref(cur))
    del g
