"""Pins for the fp64 CPU oracle, each independent of the oracle's own code.

The pages print no worked example of this path's outputs, so the oracle is
pinned by:
  * brute force on tiny inputs: exact rational dot products (fractions),
    exp without max-shift, math.fsum, and a page table expanded token by
    token here, not by the oracle;
  * a library special case: with an identity page table the result is plain
    MQA softmax attention, computed with numpy matmuls and scipy's
    softmax / logsumexp;
  * closed forms: kv_len = 1 (O is the ckv row), kv_len = 2 (a sigmoid
    blend), q = 0 (O is the mean, LSE = ln L);
  * invariants: a shift through the kpe path, token duplication (+ln 2),
    page-table permutation (bit-identical), head / request permutation,
    convexity, and split-KV partials merged by combine() = the unsplit result;
  * decoders checked over every code against torch's bf16 / float8_e4m3fn
    conversions and numpy's int8.
A planted-mistake test recompiles the oracle with typical errors and checks
that these pins catch each one.
"""
import math
import os
import re
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

SM = synth.SM_SCALE_192


# ----------------------------------------------------------------- helpers
def _dec_tensor(codes, kv_dtype):
    """Decode with library conversions (not the oracle's decoders)."""
    if kv_dtype == synth.KV_FP16:
        return np.ascontiguousarray(codes).view(np.float16).astype(np.float64)
    if kv_dtype == synth.KV_BF16 or codes.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(
            torch.bfloat16).to(torch.float64).numpy()
    if kv_dtype == synth.KV_FP8_E4M3:
        return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
            torch.float64).numpy()
    return np.ascontiguousarray(codes).view(np.int8).astype(np.float64)


def _tokens(inp, b):
    """Physical (page, slot) of every token of request b, expanded here."""
    P = inp.page_size
    pages = inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]]
    out = []
    for j, pg in enumerate(pages):
        n_slots = int(inp.kv_last_page_len[b]) if j == len(pages) - 1 else P
        for s in range(n_slots):
            out.append((int(pg), s))
    return out


def _token_rows(inp, b):
    # 644-byte layouts ("FlashMLA Ampere v2", "What is added": 644 bytes per
    # token = 512 8-bit ckv + 128 bf16 kpe + 4 scale): the scale is ckv's only
    code_dt = {synth.KV_FP8_KPE16: synth.KV_FP8_E4M3,
               synth.KV_INT8_KPE16: synth.KV_INT8}.get(inp.kv_dtype, inp.kv_dtype)
    kpe16 = inp.kv_dtype in (synth.KV_FP8_KPE16, synth.KV_INT8_KPE16)
    ck = _dec_tensor(inp.ckv, code_dt)
    kp = _dec_tensor(inp.kpe, synth.KV_BF16 if kpe16 else code_dt)
    K, R = [], []
    for pg, s in _tokens(inp, b):
        sig = 1.0 if inp.kv_scale is None else float(inp.kv_scale[pg, s])
        K.append(ck[pg, s] * sig)
        R.append(kp[pg, s] * (1.0 if kpe16 else sig))
    return np.array(K).reshape(-1, 512), np.array(R).reshape(-1, 64)


def brute_force(inp):
    """Exact-rational scores, exp without max-shift, fsum.  With qo_len = q
    queries per request, query i (row b * q + i) sees the first L_b - (q - 1 - i)
    tokens: the queries are the request's last q positions ("FlashMLA SM100",
    forward kernel notes: causal mask with Q at the end of the matrix)."""
    B, H, Q = inp.batch, inp.num_heads, inp.qo_len
    q16 = synth.KV_FP16 if inp.kv_dtype == synth.KV_FP16 else synth.KV_BF16
    qn = _dec_tensor(inp.q_nope, q16)
    qp = _dec_tensor(inp.q_pe, q16)
    O = np.zeros((B * Q, H, 512))
    LSE = np.zeros((B * Q, H))
    smf = Fraction(inp.sm_scale)
    for b in range(B):
        K, R = _token_rows(inp, b)
        Kf = [[Fraction(float(x)) for x in np.concatenate([K[t], R[t]])] for t in range(K.shape[0])]
        for qi in range(Q):
            row = b * Q + qi
            V = max(0, K.shape[0] - (Q - 1 - qi))
            if V == 0:
                LSE[row, :] = -np.inf
                continue
            for h in range(H):
                q = [Fraction(float(x)) for x in np.concatenate([qn[row, h], qp[row, h]])]
                s = [float(smf * sum(a * c for a, c in zip(q, Kf[t]))) for t in range(V)]
                w = [math.exp(x) for x in s]
                Z = math.fsum(w)
                LSE[row, h] = math.log(Z)
                for i in range(512):
                    O[row, h, i] = math.fsum(w[t] * K[t, i] for t in range(V)) / Z
    return O, LSE


def run_oracle(inp, rows=None, threads=4):
    return oracle.decode(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices,
                         inp.kv_last_page_len, inp.sm_scale, inp.page_size, inp.kv_dtype,
                         inp.kv_scale, rows=rows, threads=threads, qo_len=inp.qo_len)


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _close(a, b, rel=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    scale = max(1.0, float(np.abs(b[fin]).max()) if fin.any() else 1.0)
    err = float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0
    assert err <= rel * scale, err


# ------------------------------------------------------------------ decoders
def test_decode_bf16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _dec_tensor(codes, synth.KV_BF16)
    for c in range(65536):
        v = oracle.dec_bf16(c)
        assert (math.isnan(v) and math.isnan(ref[c])) or v == ref[c], c


def test_decode_e4m3fn_all_codes():
    ref = _dec_tensor(np.arange(256, dtype=np.uint8), synth.KV_FP8_E4M3)
    for c in range(256):
        v = oracle.dec_e4m3fn(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    assert oracle.dec_e4m3fn(0x7E) == 448.0 and oracle.dec_e4m3fn(0xFE) == -448.0
    assert oracle.dec_e4m3fn(0x01) == 2.0 ** -9


def test_decode_fp16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    for c in range(65536):
        v = oracle.dec_fp16(c)
        assert (math.isnan(v) and math.isnan(ref[c])) or v == ref[c], c
    assert oracle.dec_fp16(0x7BFF) == 65504.0 and oracle.dec_fp16(0x0001) == 2.0 ** -24


def test_decode_int8_all_codes():
    for c in range(256):
        assert oracle.dec_int8(c) == float(np.array([c], np.uint8).view(np.int8)[0])


# --------------------------------------------------------------- brute force
BRUTE_CASES = [
    # lengths, H, P, kv_dtype, seed
    ([5, 1, 13], 2, 4, synth.KV_BF16, 11),
    ([7, 0, 3], 3, 2, synth.KV_BF16, 12),
    ([9], 4, 1, synth.KV_BF16, 13),
    ([40, 17], 2, 16, synth.KV_BF16, 14),
    ([6, 11], 2, 4, synth.KV_FP8_E4M3, 15),
    ([10, 3], 2, 4, synth.KV_INT8, 16),
    ([7, 12], 2, 4, synth.KV_FP8_KPE16, 17),
    ([9, 2], 2, 4, synth.KV_INT8_KPE16, 18),
    ([8, 0, 13], 3, 4, synth.KV_FP16, 19),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force_tiny(case):
    lengths, H, P, kvd, seed = case
    inp = synth.make_inputs(lengths, H, P, kvd, seed=seed, poison=True, extra_pages=2)
    o, lse = run_oracle(inp)
    O, LSE = brute_force(inp)
    _close(o, O)
    _close(lse, LSE)


# --------------------------------------------- several queries per request
# (lengths, H, P, kv_dtype, seed, qo_len): short requests (L_b < qo_len) leave
# the first queries with nothing visible; an empty request leaves all of them.
CAUSAL_CASES = [
    ([5, 1, 13], 2, 4, synth.KV_BF16, 21, 3),
    ([9, 0, 4], 2, 2, synth.KV_FP8_E4M3, 22, 2),
    ([17, 6], 2, 16, synth.KV_INT8, 23, 4),
]


@pytest.mark.parametrize("case", CAUSAL_CASES)
def test_brute_force_causal_queries(case):
    lengths, H, P, kvd, seed, q = case
    inp = synth.make_inputs(lengths, H, P, kvd, seed=seed, poison=True, extra_pages=2, qo_len=q)
    o, lse = run_oracle(inp)
    O, LSE = brute_force(inp)
    _close(o, O)
    _close(lse, LSE)


def _truncated(inp, b, V):
    """Request b alone with a page table cut to its first V tokens (built here)."""
    P = inp.page_size
    one = synth.make_inputs([1], inp.num_heads, P, inp.kv_dtype, seed=0)
    one.ckv, one.kpe, one.kv_scale = inp.ckv, inp.kpe, inp.kv_scale
    n = (V + P - 1) // P
    pages = inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b] + n]
    one.kv_indptr = np.array([0, n], np.int32)
    one.kv_indices = pages.copy()
    one.kv_last_page_len = np.array([V - (n - 1) * P if n else 1], np.int32)
    one.lengths = np.array([V], np.int64)
    return one


@pytest.mark.parametrize("kvd", [synth.KV_BF16, synth.KV_FP8_E4M3])
def test_causal_query_is_decode_of_its_prefix(kvd):
    # query i of q sees exactly what a one-query decode of the request cut to
    # L_b - (q - 1 - i) tokens sees; the last query sees the whole request
    q = 4
    inp = synth.make_inputs([37, 50], 3, 16, kvd, seed=24, poison=True, qo_len=q)
    o, lse = run_oracle(inp)
    for b in range(2):
        L = int(inp.lengths[b])
        for qi in range(q):
            one = _truncated(inp, b, L - (q - 1 - qi))
            one.q_nope = inp.q_nope[b * q + qi:b * q + qi + 1]
            one.q_pe = inp.q_pe[b * q + qi:b * q + qi + 1]
            o1, l1 = run_oracle(one)
            assert np.array_equal(o1[0], o[b * q + qi]) and np.array_equal(l1[0], lse[b * q + qi])
    # the mask matters: query 0 over the whole request is a different result
    whole = _truncated(inp, 0, 37)
    whole.q_nope, whole.q_pe = inp.q_nope[0:1], inp.q_pe[0:1]
    assert not np.array_equal(run_oracle(whole)[1][0], lse[0])


def test_causal_split_partials_combine_to_unsplit():
    q, L = 3, 70
    inp = synth.make_inputs([L], 2, 16, synth.KV_BF16, seed=25, qo_len=q)
    o, lse = run_oracle(inp)
    args = (inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices,
            inp.kv_last_page_len, inp.sm_scale, inp.page_size)
    # cuts inside the masked tail: the last chunk is fully masked for query 0
    for bounds in ([0, 32, 68, 70], [0, 69, 70], [0, 16, 48, 64, 70]):
        for qi in range(q):
            for h in range(2):
                parts = [oracle.partial(*args, 0, h, bounds[i], bounds[i + 1], qo_len=q, qi=qi)
                         for i in range(len(bounds) - 1)]
                oc, lc = oracle.combine(np.array([p[1] for p in parts]),
                                        np.stack([p[0] for p in parts]))
                _close(oc, o[qi, h], 1e-12)
                assert abs(lc - lse[qi, h]) <= 1e-12 * abs(lse[qi, h])
    # a chunk past the causal limit is empty
    _, l_empty = oracle.partial(*args, 0, 0, 68, 70, qo_len=q, qi=0)
    assert l_empty == -np.inf


# ----------------------------------------------------------- library special
def test_identity_table_equals_library_mqa():
    L, H = 300, 8
    inp = synth.make_inputs([L], H, L, seed=21)
    inp.kv_indptr = np.array([0, 1], np.int32)
    inp.kv_indices = np.array([0], np.int32)
    inp.kv_last_page_len = np.array([L], np.int32)
    inp.ckv = inp.ckv[:1]
    inp.kpe = inp.kpe[:1]
    qn = _dec_tensor(inp.q_nope, 0)[0]
    qp = _dec_tensor(inp.q_pe, 0)[0]
    ck = _dec_tensor(inp.ckv, 0)[0]
    kp = _dec_tensor(inp.kpe, 0)[0]
    S = inp.sm_scale * (np.concatenate([qn, qp], 1) @ np.concatenate([ck, kp], 1).T)
    Oref = scipy.special.softmax(S, axis=1) @ ck
    LSEref = scipy.special.logsumexp(S, axis=1)
    o, lse = run_oracle(inp)
    _close(o[0], Oref, 1e-12)
    _close(lse[0], LSEref, 1e-12)


# --------------------------------------------------------------- closed forms
def test_kv_len_one_is_the_row():
    inp = synth.make_inputs([1, 1, 1], 4, 16, seed=31, poison=True)
    o, lse = run_oracle(inp)
    for b in range(3):
        K, R = _token_rows(inp, b)
        qn = _dec_tensor(inp.q_nope, 0)[b]
        qp = _dec_tensor(inp.q_pe, 0)[b]
        for h in range(4):
            assert np.array_equal(o[b, h], K[0])  # exp(0)/1 = 1 exactly
            s = inp.sm_scale * float(np.dot(qn[h], K[0]) + np.dot(qp[h], R[0]))
            assert abs(lse[b, h] - s) <= 1e-12 * max(1, abs(s))


def test_kv_len_two_sigmoid():
    inp = synth.make_inputs([2], 3, 4, seed=32)
    o, lse = run_oracle(inp)
    K, R = _token_rows(inp, 0)
    qn = _dec_tensor(inp.q_nope, 0)[0]
    qp = _dec_tensor(inp.q_pe, 0)[0]
    for h in range(3):
        s0 = inp.sm_scale * (qn[h] @ K[0] + qp[h] @ R[0])
        s1 = inp.sm_scale * (qn[h] @ K[1] + qp[h] @ R[1])
        sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
        _close(o[0, h], sig * K[1] + (1 - sig) * K[0], 1e-12)
        assert abs(lse[0, h] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-12 * 10


@pytest.mark.parametrize("kvd", [synth.KV_BF16, synth.KV_FP8_E4M3, synth.KV_INT8])
def test_zero_query_gives_mean_and_log_len(kvd):
    lengths = [37, 64, 5]
    inp = synth.make_inputs(lengths, 2, 16, kvd, seed=33, poison=True)
    inp.q_nope[:] = 0
    inp.q_pe[:] = 0
    o, lse = run_oracle(inp)
    for b, L in enumerate(lengths):
        K, _ = _token_rows(inp, b)
        mean = np.array([math.fsum(K[:, i]) / L for i in range(512)])
        for h in range(2):
            _close(o[b, h], mean, 1e-13)
            assert abs(lse[b, h] - math.log(L)) < 1e-13


# ---------------------------------------------------------------- invariants
def test_shift_through_kpe_path():
    inp = synth.make_inputs([50, 23], 4, 16, seed=34)
    one = _bf16(1.0)[()]
    inp.kpe[..., 0] = one
    inp.q_pe[..., 0] = 0
    o0, l0 = run_oracle(inp)
    c = 2.0
    inp.q_pe[..., 0] = _bf16(c)[()]
    o1, l1 = run_oracle(inp)
    _close(o1, o0, 1e-12)
    _close(l1 - l0, np.full_like(l0, inp.sm_scale * c), 1e-12)


def test_duplicating_every_token_adds_ln2():
    base = synth.make_inputs([19], 3, 1, seed=35)
    o0, l0 = run_oracle(base)
    dup = synth.make_inputs([19], 3, 1, seed=35)
    idx = base.kv_indices
    dup.kv_indices = np.repeat(idx, 2).astype(np.int32)
    dup.kv_indptr = np.array([0, 2 * idx.size], np.int32)
    o1, l1 = run_oracle(dup)
    _close(o1, o0, 1e-12)
    _close(l1 - l0, np.full_like(l0, math.log(2.0)), 1e-12)


def test_page_permutation_is_bit_identical():
    inp = synth.make_inputs([70, 33, 100], 4, 16, seed=36, extra_pages=3)
    o0, l0 = run_oracle(inp)
    rng = np.random.default_rng(7)
    perm = rng.permutation(inp.num_pages)  # new position of each old page
    ck = np.empty_like(inp.ckv)
    kp = np.empty_like(inp.kpe)
    ck[perm] = inp.ckv
    kp[perm] = inp.kpe
    inp.ckv, inp.kpe = ck, kp
    inp.kv_indices = perm[inp.kv_indices].astype(np.int32)
    o1, l1 = run_oracle(inp)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_head_and_request_permutation():
    inp = synth.make_inputs([20, 45, 9], 5, 4, seed=37)
    o0, l0 = run_oracle(inp)
    hp = np.array([3, 0, 4, 1, 2])
    inp2 = synth.make_inputs([20, 45, 9], 5, 4, seed=37)
    inp2.q_nope = inp.q_nope[:, hp].copy()
    inp2.q_pe = inp.q_pe[:, hp].copy()
    o1, l1 = run_oracle(inp2)
    assert np.array_equal(o1, o0[:, hp]) and np.array_equal(l1, l0[:, hp])
    # requests in reverse order, same pages
    rp = [2, 1, 0]
    segs = [inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]] for b in rp]
    inp3 = synth.make_inputs([20, 45, 9], 5, 4, seed=37)
    inp3.kv_indices = np.concatenate(segs).astype(np.int32)
    inp3.kv_indptr = np.concatenate([[0], np.cumsum([s.size for s in segs])]).astype(np.int32)
    inp3.kv_last_page_len = inp.kv_last_page_len[rp].copy()
    inp3.q_nope = inp.q_nope[rp].copy()
    inp3.q_pe = inp.q_pe[rp].copy()
    o2, l2 = run_oracle(inp3)
    assert np.array_equal(o2, o0[rp]) and np.array_equal(l2, l0[rp])


def test_convexity():
    inp = synth.make_inputs([64, 3], 4, 16, synth.KV_FP8_E4M3, seed=38)
    o, _ = run_oracle(inp)
    for b in range(2):
        K, _ = _token_rows(inp, b)
        lo, hi = K.min(0), K.max(0)
        eps = 1e-12 * np.abs(K).max()
        assert np.all(o[b] >= lo - eps) and np.all(o[b] <= hi + eps)


@pytest.mark.parametrize("kvd", [synth.KV_BF16, synth.KV_INT8])
def test_split_partials_combine_to_unsplit(kvd):
    L = 130
    inp = synth.make_inputs([L, 77], 3, 16, kvd, seed=39)
    o, lse = run_oracle(inp)
    rng = np.random.default_rng(3)
    args = (inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices,
            inp.kv_last_page_len, inp.sm_scale, inp.page_size)
    for trial in range(4):
        cuts = np.sort(rng.choice(np.arange(1, L), size=trial + 1, replace=False))
        bounds = [0] + list(cuts) + [L]
        if trial == 3:
            bounds = [0, 0] + bounds[1:]  # an empty chunk carries no weight
        for h in range(3):
            parts = [oracle.partial(*args, 0, h, bounds[i], bounds[i + 1], kvd, inp.kv_scale)
                     for i in range(len(bounds) - 1)]
            oc, lc = oracle.combine(np.array([p[1] for p in parts]),
                                    np.stack([p[0] for p in parts]))
            _close(oc, o[0, h], 1e-12)
            assert abs(lc - lse[0, h]) <= 1e-12 * abs(lse[0, h])


def test_empty_request_and_neighbours():
    inp = synth.make_inputs([12, 0, 12], 2, 4, seed=40)
    o, lse = run_oracle(inp)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    assert oracle.kv_len(inp.kv_indptr, inp.kv_last_page_len, 4, 1) == 0
    assert oracle.kv_len(inp.kv_indptr, inp.kv_last_page_len, 4, 2) == 12
    # the neighbours are what they are without the empty request in between
    for b in (0, 2):
        one = synth.make_inputs([12, 0, 12], 2, 4, seed=40)
        one.q_nope, one.q_pe = inp.q_nope[b:b + 1], inp.q_pe[b:b + 1]
        one.kv_indptr = np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]], np.int32)
        one.kv_indices = inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]].copy()
        one.kv_last_page_len = inp.kv_last_page_len[b:b + 1].copy()
        o1, l1 = run_oracle(one)
        assert np.array_equal(o1[0], o[b]) and np.array_equal(l1[0], lse[b])


def test_last_page_len_bounds_the_tokens():
    # 3 pages of 16 with 5 valid slots in the last page: L = 37; poisoned tail
    inp = synth.make_inputs([37], 2, 16, seed=41, poison=True)
    assert int(inp.kv_last_page_len[0]) == 5
    assert oracle.kv_len(inp.kv_indptr, inp.kv_last_page_len, 16, 0) == 37
    o, lse = run_oracle(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_row_selection_matches_full_and_thread_count():
    inp = synth.make_inputs([33, 70, 5, 18], 4, 16, seed=42)
    o, lse = run_oracle(inp, threads=3)
    o1, l1 = run_oracle(inp, threads=1)
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    rows = np.array([15, 0, 6, 9], np.int32)
    orow, lrow = run_oracle(inp, rows=rows, threads=2)
    assert np.array_equal(orow, o.reshape(-1, 512)[rows])
    assert np.array_equal(lrow, lse.reshape(-1)[rows])


# ----------------------------------------------------- planted-mistake check
# ---- quantisation on cache append (oracle.quantize / oracle.enc_e4m3fn) ----
# The reading: scale = max|x| / 448 (e4m3) or / 127 (int8) in binary32 (1 for an
# all-zero token), code = nearest representable value of x / scale (binary32
# division), ties to even, saturated; "FlashMLA Ampere v2", "What is added"
# (8-bit cache with one scale per token).

def _e4m3_values():
    return [(c, oracle.dec_e4m3fn(c)) for c in range(256) if c not in (0x7F, 0xFF)]


def test_encode_e4m3fn_round_trips_every_code():
    for c, v in _e4m3_values():
        assert oracle.enc_e4m3fn(v) == c, (hex(c), v)


def test_encode_e4m3fn_ties_go_to_even_mantissa():
    pos = sorted(v for c, v in _e4m3_values() if c < 0x80)
    for lo, hi in zip(pos, pos[1:]):
        mid = (lo + hi) / 2  # exact in binary32 for e4m3 neighbours
        c = oracle.enc_e4m3fn(mid)
        assert c % 2 == 0 and oracle.dec_e4m3fn(c) in (lo, hi), (lo, hi, hex(c))
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(1000))
        assert oracle.dec_e4m3fn(oracle.enc_e4m3fn(float(below))) == lo
        assert oracle.dec_e4m3fn(oracle.enc_e4m3fn(float(above))) == hi


def test_encode_e4m3fn_matches_library_rounding():
    # library special case: torch's float32 -> float8_e4m3fn conversion (round to
    # nearest even) on values inside the finite range
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000) * 2.0 ** rng.integers(-12, 8, 4000),
                        [v for _, v in _e4m3_values()]]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.enc_e4m3fn(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_encode_e4m3fn_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38):
        assert oracle.enc_e4m3fn(v) == 0x7E and oracle.enc_e4m3fn(-v) == 0xFE


def _bf16(x):
    x = np.asarray(x, np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # exact for bf16-representable x


def test_quantize_scale_and_codes_definition():
    rng = np.random.default_rng(3)
    n = 40
    xf = (rng.normal(0, 1, (n, 576)) * 2.0 ** rng.integers(-20, 10, (n, 1))).astype(np.float32)
    xb = _bf16(xf)
    x = (xb.astype(np.uint32) << 16).view(np.float32)
    for kvd, qmax in ((oracle.KV_FP8_E4M3, 448.0), (oracle.KV_INT8, 127.0)):
        cc, kc, sc = oracle.quantize(xb[:, :512], xb[:, 512:], kvd)
        codes = np.concatenate([cc, kc], axis=1)
        amax = np.abs(x).max(axis=1)
        assert np.array_equal(sc, (amax / np.float32(qmax)).astype(np.float32))
        dec = oracle.dec_e4m3fn if kvd == oracle.KV_FP8_E4M3 else oracle.dec_int8
        for j in range(n):
            v = x[j] / sc[j]  # binary32, as the definition
            back = np.array([dec(c) for c in codes[j]])
            if kvd == oracle.KV_INT8:
                assert np.array_equal(back, np.clip(np.rint(v), -127, 127))
            else:
                # nearest representable: no e4m3 value is strictly closer
                grid = np.array(sorted(v2 for _, v2 in _e4m3_values()))
                err = np.abs(back - v)
                best = np.abs(grid[None, :] - v[:, None]).min(axis=1)
                assert np.all(err <= best)
            # the largest magnitude maps to the end of the range
            assert np.abs(back).max() == qmax


@pytest.mark.parametrize("kvd", [synth.KV_FP8_KPE16, synth.KV_INT8_KPE16])
def test_quantize_644_record_scales_ckv_only(kvd):
    # "FlashMLA Ampere v2", "What is added": 644 bytes per token = 512 8-bit
    # ckv codes + 64 bf16 kpe + one fp32 scale, so kpe is not quantised and
    # the scale is set by ckv alone; a kpe value far above every ckv value
    # must not change the scale or the codes
    rng = np.random.default_rng(77)
    c = rng.normal(0, 1, (5, 512)).astype(np.float32)
    k = rng.normal(0, 1, (5, 64)).astype(np.float32)
    k[:, 3] = 1e4
    cb, kb = _bf16(c), _bf16(k)
    cc, kc, sc = oracle.quantize(cb, kb, kvd)
    assert np.array_equal(kc, kb)
    qmax = np.float32(448.0 if kvd == synth.KV_FP8_KPE16 else 127.0)
    cf = (cb.astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(cf).max(axis=1)
    assert np.array_equal(sc, (amax / qmax).astype(np.float32))
    full = synth.KV_FP8_E4M3 if kvd == synth.KV_FP8_KPE16 else synth.KV_INT8
    cc2, _, sc2 = oracle.quantize(cb, np.zeros_like(kb), full)  # kpe of zeros: same amax
    assert np.array_equal(cc, cc2) and np.array_equal(sc, sc2)


def test_quantize_all_zero_token():
    z = np.zeros((2, 576), np.uint16)
    z[1, 7] = 0x8000  # -0.0
    for kvd in (oracle.KV_FP8_E4M3, oracle.KV_INT8):
        cc, kc, sc = oracle.quantize(z[:, :512], z[:, 512:], kvd)
        assert np.all(sc == 1.0)
        assert all(c in (0, 0x80) for c in np.concatenate([cc.ravel(), kc.ravel()]))


def test_quantize_error_bound():
    # |dec(code) * scale - x| <= half a grid step at |x / scale| times the scale
    rng = np.random.default_rng(8)
    xb = _bf16(rng.normal(0, 1, (16, 576)).astype(np.float32))
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cc, kc, sc = oracle.quantize(xb[:, :512], xb[:, 512:], oracle.KV_FP8_E4M3)
    codes = np.concatenate([cc, kc], axis=1)
    back = np.vectorize(oracle.dec_e4m3fn)(codes) * sc[:, None].astype(np.float64)
    v = np.abs(x / sc[:, None])
    step = np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3))
    assert np.all(np.abs(back - x) <= 0.5 * step * sc[:, None] * (1 + 1e-6))


PIN_SUITE = [
    lambda: test_brute_force_tiny(BRUTE_CASES[0]),
    lambda: test_brute_force_tiny(BRUTE_CASES[4]),
    lambda: test_brute_force_tiny(BRUTE_CASES[5]),
    test_identity_table_equals_library_mqa,
    test_kv_len_one_is_the_row,
    lambda: test_zero_query_gives_mean_and_log_len(synth.KV_FP8_E4M3),
    test_shift_through_kpe_path,
    lambda: test_split_partials_combine_to_unsplit(synth.KV_BF16),
    test_decode_e4m3fn_all_codes,
    test_decode_int8_all_codes,
    test_last_page_len_bounds_the_tokens,
    test_encode_e4m3fn_round_trips_every_code,
    test_encode_e4m3fn_ties_go_to_even_mantissa,
    test_encode_e4m3fn_saturates,
    test_quantize_scale_and_codes_definition,
    lambda: test_brute_force_causal_queries(CAUSAL_CASES[0]),
    lambda: test_brute_force_tiny(BRUTE_CASES[6]),
    lambda: test_brute_force_tiny(BRUTE_CASES[8]),
    test_decode_fp16_all_codes,
    lambda: test_brute_force_tiny(BRUTE_CASES[7]),
    lambda: test_quantize_644_record_scales_ckv_only(synth.KV_FP8_KPE16),
    lambda: test_causal_query_is_decode_of_its_prefix(synth.KV_BF16),
]

MUTANTS = {
    "drop_kpe_term": ("for (i = 0; i < D_KPE; ++i) dot += q[D_CKV + i] * R[i];", ""),
    "slot_index": ("int64_t slot = t % P;", "int64_t slot = (t + 1) % P;"),
    "no_sm_scale": ("s[t] = in->sm_scale * dot;", "s[t] = dot;"),
    "lse_without_max": ("*lse = m + log(Z);", "*lse = log(Z);"),
    "kv_len_full_pages": ("return (n - 1) * (int64_t)page_size + (int64_t)kv_last_page_len[b];",
                          "return n * (int64_t)page_size;"),
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "int8_unsigned": ("return (double)(int8_t)code;", "return (double)code;"),
    "kpe_unscaled": ("oracle_dec_int8(k[i])) * sigma;", "oracle_dec_int8(k[i]));"),
    "combine_weight": ("double w = exp(lse_parts[i] - lse);", "double w = exp(lse_parts[i] - M);"),
    "value_from_wrong_head": ("(qrow * in->num_heads + h) * D_CKV;",
                              "(qrow * in->num_heads + 0) * D_CKV;"),
    "unnormalised": ("double p = exp(s[t] - m) / Z;", "double p = exp(s[t] - m);"),
    "encode_ties_up": ("r = nearbyint(a / ldexp(1.0, E - 3)); /* 8 .. 16 */",
                       "r = floor(a / ldexp(1.0, E - 3) + 0.5);"),
    "encode_no_saturation": ("if (a >= 448.0) {", "if (a >= 1e30) {"),
    "encode_exponent": ("code = ((E + 7) << 3) | ((int)r - 8);", "code = ((E + 8) << 3) | ((int)r - 8);"),
    "quant_scale_int8": ("ckv_fp8(kv_dtype) ? 448.0f : 127.0f;", "ckv_fp8(kv_dtype) ? 448.0f : 128.0f;"),
    "quant_truncate": ("float r = nearbyintf(v);", "float r = truncf(v);"),
    "causal_off_by_one": ("(int64_t)(in->qo_len - 1 - qi);", "(int64_t)(in->qo_len - qi);"),
    "causal_reversed": ("(int64_t)(in->qo_len - 1 - qi);", "(int64_t)(qi);"),
    "causal_none": ("(int64_t)(in->qo_len - 1 - qi);", "(int64_t)0;"),
    "query_row_ignores_index": ("const int64_t qrow = (int64_t)b * in->qo_len + qi;",
                                "const int64_t qrow = (int64_t)b * in->qo_len;"),
    "kpe16_scaled": ("row * D_KPE;\n    for (i = 0; i < D_KPE; ++i) R[i] = oracle_dec_bf16(k[i]);\n  } else",
                     "row * D_KPE;\n    for (i = 0; i < D_KPE; ++i) R[i] = oracle_dec_bf16(k[i]) * sigma;\n  } else"),
    "kpe16_amax_over_kpe": ("const int nq = kpe_bf16(kv_dtype) ? D_CKV : D_CKV + D_KPE;",
                            "const int nq = D_CKV + D_KPE;"),
    "fp16_bias": ("ldexp(1.0 + (double)m / 1024.0, e - 15)", "ldexp(1.0 + (double)m / 1024.0, e - 16)"),
    "fp16_queries_as_bf16": ("for (i = 0; i < D_CKV; ++i) q[i] = dec16(in->kv_dtype, qn[i]);",
                             "for (i = 0; i < D_CKV; ++i) q[i] = oracle_dec_bf16(qn[i]);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")).read()
    assert src.count(old) == 1, name
    mutant = src.replace(old, new)
    tmp = tempfile.mkdtemp()
    try:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as f:
            f.write(mutant)
        so = os.path.join(tmp, "libmutant.so")
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", path, "-o",
                               so, "-lm"])
        saved_lib, saved_path = oracle._lib, oracle._LIB
        try:
            oracle._lib = None
            oracle._LIB = so
            oracle._SRC = path
            caught = 0
            for pin in PIN_SUITE:
                try:
                    pin()
                except (AssertionError, RuntimeError):
                    caught += 1
            assert caught > 0, "mutant %s survived every pin" % name
        finally:
            oracle._lib, oracle._LIB = saved_lib, saved_path
            oracle._SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_bf16_token_record_is_1152_bytes():
    # "FlashMLA Ampere v2", "What is added": the bf16 latent token takes 1152 bytes
    # (512 ckv + 64 kpe values, 2 bytes each); the 8-bit record the pages describe is
    # 644 bytes and their ideal speed-up 1152 / 644 = 1.79 ("Performance").
    inp = synth.make_inputs([3], 16, 16, seed=1)
    assert inp.kv_bytes_per_token() == 1152
    assert round(1152 / 644, 2) == 1.79
