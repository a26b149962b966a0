"""GPU tests of mla_cache_append (cache append with quantisation on write)
against the oracle.  Copies (bf16) and 8-bit codes and scales must be
bit-exact: both sides take every rounding decision in binary32 (the reading
stated in the oracle), so there is one right answer.  Rows not named by
`slots` must be left untouched."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_decode_amd as mla
    mla.load_library()


def _tokens(n, seed, wide=False):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (n, 576)).astype(np.float32)
    if wide:  # per-token magnitudes across many binades, plus exact zeros
        x *= (2.0 ** rng.integers(-30, 30, (n, 1))).astype(np.float32)
        x[rng.random((n, 576)) < 0.05] = 0.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern works
    if n > 2:
        bits[0] = 0          # all-zero token
        bits[1, :] = 0
        bits[1, 3] = 0x8000  # -0.0 and one tiny value
        bits[1, 4] = 0x0001
    return bits


def _dev_bf16(bits, fp16=False):
    return torch.from_numpy(bits.view(np.int16)).view(
        torch.float16 if fp16 else torch.bfloat16).cuda()


def _cache(pages, P, kv_dtype, seed):
    rng = np.random.default_rng(seed)
    kpe16 = kv_dtype in (synth.KV_FP8_KPE16, synth.KV_INT8_KPE16)
    if kv_dtype in (synth.KV_BF16, synth.KV_FP16):
        t16 = torch.float16 if kv_dtype == synth.KV_FP16 else torch.bfloat16
        ckv = torch.from_numpy(rng.integers(0, 65536, (pages, P, 512)).astype(np.uint16).view(
            np.int16)).view(t16).cuda()
        kpe = torch.from_numpy(rng.integers(0, 65536, (pages, P, 64)).astype(np.uint16).view(
            np.int16)).view(t16).cuda()
        return ckv, kpe, None
    ckv = torch.from_numpy(rng.integers(0, 256, (pages, P, 512)).astype(np.uint8)).cuda()
    if kpe16:
        kpe = torch.from_numpy(rng.integers(0, 65536, (pages, P, 64)).astype(np.uint16).view(
            np.int16)).view(torch.bfloat16).cuda()
    else:
        kpe = torch.from_numpy(rng.integers(0, 256, (pages, P, 64)).astype(np.uint8)).cuda()
    sc = torch.from_numpy(rng.normal(0, 1, (pages, P)).astype(np.float32)).cuda()
    return ckv, kpe, sc


def _as_u(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16) \
        if t.dtype in (torch.bfloat16, torch.float16) else t.cpu().numpy()


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8_E4M3, synth.KV_INT8,
                                      synth.KV_FP8_KPE16, synth.KV_INT8_KPE16, synth.KV_FP16])
@pytest.mark.parametrize("n,wide", [(1, False), (37, False), (1000, True), (4099, False)])
def test_append_matches_oracle(kv_dtype, n, wide):
    import mla_paged_kv_decode_amd as mla
    pages, P = (n + 63) // 64 + 3, 64
    bits = _tokens(n, seed=n + kv_dtype, wide=wide)
    rng = np.random.default_rng(n)
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    slots[rng.random(n) < 0.1] = -1  # padding tokens are skipped
    ckv, kpe, sc = _cache(pages, P, kv_dtype, seed=n)
    before = [_as_u(ckv).copy(), _as_u(kpe).copy(), None if sc is None else sc.cpu().numpy()]
    print("case kv_dtype=%d n=%d" % (kv_dtype, n), flush=True)
    f16 = kv_dtype == synth.KV_FP16  # a copy: any 16-bit pattern
    mla.cache_append(_dev_bf16(bits[:, :512].copy(), f16), _dev_bf16(bits[:, 512:].copy(), f16),
                     torch.from_numpy(slots).cuda(), ckv, kpe, kv_dtype, sc)
    torch.cuda.synchronize()
    got_c = _as_u(ckv).reshape(pages * P, 512)
    got_k = _as_u(kpe).reshape(pages * P, 64)
    exp_c = before[0].reshape(pages * P, 512).copy()
    exp_k = before[1].reshape(pages * P, 64).copy()
    live = slots >= 0
    if kv_dtype in (synth.KV_BF16, synth.KV_FP16):
        exp_c[slots[live]] = bits[live, :512]
        exp_k[slots[live]] = bits[live, 512:]
    else:
        cc, kc, s = oracle.quantize(bits[:, :512], bits[:, 512:], kv_dtype)
        exp_c[slots[live]] = cc[live]
        exp_k[slots[live]] = kc[live]
        exp_s = before[2].reshape(-1).copy()
        exp_s[slots[live]] = s[live]
        got_s = sc.cpu().numpy().reshape(-1)
        assert np.array_equal(got_s.view(np.uint32), exp_s.view(np.uint32))
    assert np.array_equal(got_c, exp_c)
    assert np.array_equal(got_k, exp_k)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8_E4M3, synth.KV_INT8, synth.KV_FP8_KPE16,
                                      synth.KV_INT8_KPE16])
def test_append_then_decode(kv_dtype):
    """A cache built token by token with mla_cache_append decodes like the
    oracle on the oracle's quantisation of the same tokens."""
    import mla_paged_kv_decode_amd as mla
    src = synth.make_inputs([300, 1, 77, 1024], 16, 16, synth.KV_BF16, seed=31)
    P, pages = src.page_size, src.num_pages
    # tokens of every request, in order, with their cache rows
    rows, toks_c, toks_k = [], [], []
    for b in range(src.batch):
        for t in range(int(src.lengths[b])):
            page = src.kv_indices[src.kv_indptr[b] + t // P]
            rows.append(page * P + t % P)
            toks_c.append(src.ckv[page, t % P])
            toks_k.append(src.kpe[page, t % P])
    rows = np.array(rows, np.int64)
    tc, tk = np.stack(toks_c), np.stack(toks_k)
    kpe16 = kv_dtype in (synth.KV_FP8_KPE16, synth.KV_INT8_KPE16)
    ckv = torch.zeros((pages, P, 512), dtype=torch.uint8, device="cuda")
    kpe = torch.zeros((pages, P, 64), dtype=torch.bfloat16 if kpe16 else torch.uint8,
                      device="cuda")
    sc = torch.ones((pages, P), dtype=torch.float32, device="cuda")
    mla.cache_append(_dev_bf16(tc), _dev_bf16(tk), torch.from_numpy(rows).cuda(), ckv, kpe,
                     kv_dtype, sc)
    torch.cuda.synchronize()
    cc, kc, s = oracle.quantize(tc, tk, kv_dtype)
    ref_ckv = np.zeros((pages * P, 512), np.uint8)
    ref_kpe = np.zeros((pages * P, 64), np.uint16 if kpe16 else np.uint8)
    ref_sc = np.ones(pages * P, np.float32)
    ref_ckv[rows], ref_kpe[rows], ref_sc[rows] = cc, kc, s
    assert np.array_equal(ckv.cpu().numpy().reshape(-1, 512), ref_ckv)
    assert np.array_equal(_as_u(kpe).reshape(-1, 64), ref_kpe)
    assert np.array_equal(sc.cpu().numpy().reshape(-1), ref_sc)
    q8 = synth.MlaInputs(src.batch, src.num_heads, P, kv_dtype, src.lengths, src.q_nope, src.q_pe,
                         ref_ckv.reshape(pages, P, 512), ref_kpe.reshape(pages, P, 64),
                         ref_sc.reshape(pages, P), src.kv_indptr, src.kv_indices,
                         src.kv_last_page_len, src.sm_scale)
    qn = _dev_bf16(src.q_nope)
    qp = _dev_bf16(src.q_pe)
    ip, ix, lp = (torch.from_numpy(getattr(src, k)).cuda() for k in
                  ("kv_indptr", "kv_indices", "kv_last_page_len"))
    o, lse = mla.decode(qn, qp, ckv, kpe, ip, ix, lp, src.sm_scale, kv_dtype, sc,
                        kv_indptr_host=src.kv_indptr, kv_last_page_len_host=src.kv_last_page_len)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(q8.q_nope, q8.q_pe, q8.ckv, q8.kpe, q8.kv_indptr, q8.kv_indices,
                                   q8.kv_last_page_len, q8.sm_scale, P, kv_dtype, q8.kv_scale)
    a = o.float().cpu().numpy().astype(np.float64).ravel()
    b = o_ref.ravel()
    assert 1 - a @ b / (np.linalg.norm(a) * np.linalg.norm(b)) <= 1e-4
    assert np.abs(a - b).max() <= 2e-2
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= 1e-3
