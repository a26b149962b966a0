"""Seeded synthetic inputs for paged MLA decode.

This module only draws and lays out input data; it holds none of the decode
arithmetic, and neither the GPU path nor the oracle is imported here.  Both
sides receive the same host arrays from it.

Recipe (the inputs the pages describe, made concrete):
  * q_nope [B * qo_len, H, 512], q_pe [B * qo_len, H, 64], ckv [pages, P, 512],
    kpe [pages, P, 64] are N(0, 1) draws rounded to bf16 (round-to-nearest-even);
    qo_len = 1 for plain decode, more for several new tokens per request.  Gaussian rather
    than zero inputs, as flashinfer PR 844's review notes that zero
    initialisation inflates measured throughput.
  * Each request b has L_b tokens in n_b = ceil(L_b / P) pages; the last page
    holds L_b - (n_b - 1) * P valid slots (``kv_last_page_len``).  The page
    pool is a seeded random permutation, so a request's pages are scattered.
  * Optional poison: slots past a request's end and extra pages that no
    request references are filled with NaN codes (NaN in ``kv_scale`` for
    int8, which has no NaN code), so that any read of them shows in the output
    (FlashMLA PR 233, "Correctness": NaN padding).
  * 8-bit caches (FlashMLA PR 233, "What is added"): one fp32 scale per token
    over all 576 latent values, scale = max|x| / 448 (fp8 e4m3) or / 127
    (int8), codes = round-to-nearest-even of x / scale, saturated; a token
    whose values are all zero gets scale 1.  The 644-byte record of the same
    page (8-bit ckv, bf16 kpe, fp32 scale) quantises ckv alone, with the scale
    from its 512 values.
  * sm_scale = fp32(1 / sqrt(192)).

Random streams: numpy PCG64 generators spawned from one SeedSequence(seed),
one per tensor, so each tensor is reproducible on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

D_CKV, D_KPE = 512, 64
KV_BF16, KV_FP8_E4M3, KV_INT8 = 0, 1, 2
# 644-byte token record: 8-bit ckv codes + bf16 kpe + fp32 scale (ckv only)
KV_FP8_KPE16, KV_INT8_KPE16 = 3, 4
# fp16 cache with fp16 queries
KV_FP16 = 5
FP16_NAN = 0x7E00
KV_DTYPE_NAMES = {KV_BF16: "bf16", KV_FP8_E4M3: "fp8_e4m3", KV_INT8: "int8"}

BF16_NAN = 0x7FC0
FP8_E4M3_NAN = 0x7F
SM_SCALE_192 = float(np.float32(1.0 / math.sqrt(192.0)))


@dataclasses.dataclass
class MlaInputs:
    batch: int
    num_heads: int
    page_size: int
    kv_dtype: int
    lengths: np.ndarray           # int64 [B]
    q_nope: np.ndarray            # uint16 (bf16 bits; fp16 for KV_FP16) [B * qo_len, H, 512]
    q_pe: np.ndarray              # uint16 (bf16 bits; fp16 for KV_FP16) [B * qo_len, H, 64]
    ckv: np.ndarray               # uint16 [pages, P, 512] (bf16) or uint8 codes
    kpe: np.ndarray               # uint16 [pages, P, 64] (bf16) or uint8 codes
    kv_scale: Optional[np.ndarray]  # float32 [pages, P] for 8-bit caches, else None
    kv_indptr: np.ndarray         # int32 [B + 1]
    kv_indices: np.ndarray        # int32 [sum n_b]
    kv_last_page_len: np.ndarray  # int32 [B]
    sm_scale: float
    ckv_src: Optional[np.ndarray] = None  # bf16 source of an 8-bit cache
    kpe_src: Optional[np.ndarray] = None
    qo_len: int = 1               # queries per request (the last qo_len positions)

    @property
    def num_pages(self) -> int:
        return int(self.ckv.shape[0])

    def kv_bytes_per_token(self) -> int:
        if self.kv_dtype in (KV_BF16, KV_FP16):
            return 2 * (D_CKV + D_KPE)
        if self.kv_dtype in (KV_FP8_KPE16, KV_INT8_KPE16):
            return D_CKV + 2 * D_KPE + 4  # 644
        return D_CKV + D_KPE + 4

    def algorithmic_bytes(self) -> int:
        """Every input and output counted once, as in the nvbench accounting
        quoted on the "Benchmarking MLA" page: q_nope + q_pe + the KV rows the
        requests cover + kv_indptr + kv_indices + kv_last_page_len, plus o
        (bf16) and lse (fp32)."""
        NQ, H = self.batch * self.qo_len, self.num_heads
        q = NQ * H * (D_CKV + D_KPE) * 2
        kv = int(self.lengths.sum()) * self.kv_bytes_per_token()
        meta = 4 * (self.kv_indptr.size + self.kv_indices.size + self.kv_last_page_len.size)
        out = NQ * H * D_CKV * 2 + NQ * H * 4
        return q + kv + meta + out

    def visible_tokens(self) -> int:
        """Sum over the queries of the tokens each may attend to (causal, with
        the qo_len queries at the end of their request)."""
        q = self.qo_len
        return int(sum(max(0, int(L) - (q - 1 - i)) for L in self.lengths for i in range(q)))

    def flops(self) -> int:
        """2 * H * (576 + 512) per visible (query, token) pair: QK over 576
        dims, PV over 512."""
        return int(2 * self.num_heads * self.visible_tokens() * (D_CKV + D_KPE + D_CKV))


def _rngs(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24,
                 fp16: bool = False) -> np.ndarray:
    """N(0,1) draws rounded to bf16 (or fp16), returned as uint16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        f = rng.standard_normal(e - s, dtype=np.float32)
        if fp16:
            out[s:e] = f.astype(np.float16).view(np.uint16)
        else:
            out[s:e] = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(
                np.uint16)
    return out.reshape(shape)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _quantize_tokens(ckv_bits: np.ndarray, kpe_bits: np.ndarray, kv_dtype: int):
    """Per-token 8-bit codes and fp32 scales of a bf16 source (input recipe).
    The 644-byte layouts quantise ckv only (amax over its 512 values) and keep
    kpe as the bf16 source."""
    pages, P = ckv_bits.shape[0], ckv_bits.shape[1]
    kpe16 = kv_dtype in (KV_FP8_KPE16, KV_INT8_KPE16)
    fp8 = kv_dtype in (KV_FP8_E4M3, KV_FP8_KPE16)
    ckv_codes = np.empty(ckv_bits.shape, np.uint8)
    kpe_codes = kpe_bits.copy() if kpe16 else np.empty(kpe_bits.shape, np.uint8)
    scale = np.empty((pages, P), np.float32)
    step = max(1, (1 << 22) // (P * (D_CKV + D_KPE)))
    qmax = np.float32(448.0 if fp8 else 127.0)
    for p0 in range(0, pages, step):
        p1 = min(pages, p0 + step)
        c = _bf16_bits_to_f32(ckv_bits[p0:p1])
        k = _bf16_bits_to_f32(kpe_bits[p0:p1])
        amax = np.abs(c).max(axis=-1)
        if not kpe16:
            amax = np.maximum(amax, np.abs(k).max(axis=-1))
        s = np.where(amax > 0, amax / qmax, np.float32(1.0)).astype(np.float32)
        scale[p0:p1] = s
        for src, dst in ((c, ckv_codes),) + ((() if kpe16 else ((k, kpe_codes),))):
            y = np.clip(src / s[..., None], -qmax, qmax).astype(np.float32)
            if fp8:
                codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
                dst[p0:p1] = codes.view(torch.uint8).numpy()
            else:
                dst[p0:p1] = np.rint(y).astype(np.int8).view(np.uint8)
    return ckv_codes, kpe_codes, scale


def page_table(lengths, page_size: int, rng: np.random.Generator, extra_pages: int = 0):
    """CSR page table for the given lengths over a randomly permuted pool of
    sum(n_b) + extra_pages pages.  Returns (indptr, indices, last_len, pages)."""
    lengths = np.asarray(lengths, np.int64)
    n = (lengths + page_size - 1) // page_size
    indptr = np.zeros(lengths.size + 1, np.int64)
    indptr[1:] = np.cumsum(n)
    last = np.where(n > 0, lengths - (n - 1) * page_size, 1)
    total_pages = int(indptr[-1]) + int(extra_pages)
    perm = rng.permutation(total_pages)
    indices = perm[: int(indptr[-1])]
    return (indptr.astype(np.int32), indices.astype(np.int32), last.astype(np.int32), total_pages)


def make_inputs(lengths, num_heads: int, page_size: int, kv_dtype: int = KV_BF16, seed: int = 0,
                poison: bool = False, extra_pages: int = 0,
                sm_scale: float = SM_SCALE_192, qo_len: int = 1) -> MlaInputs:
    lengths = np.asarray(lengths, np.int64)
    B = int(lengths.size)
    H = int(num_heads)
    P = int(page_size)
    r_qn, r_qp, r_ckv, r_kpe, r_perm = _rngs(seed, 5)
    indptr, indices, last, pages = page_table(lengths, P, r_perm, extra_pages)
    f16 = kv_dtype == KV_FP16
    q_nope = _normal_bf16(r_qn, (B * qo_len, H, D_CKV), fp16=f16)
    q_pe = _normal_bf16(r_qp, (B * qo_len, H, D_KPE), fp16=f16)
    ckv = _normal_bf16(r_ckv, (pages, P, D_CKV), fp16=f16)
    kpe = _normal_bf16(r_kpe, (pages, P, D_KPE), fp16=f16)
    ckv_src = kpe_src = None
    kv_scale = None
    if kv_dtype not in (KV_BF16, KV_FP16):
        ckv_src, kpe_src = ckv, kpe
        ckv, kpe, kv_scale = _quantize_tokens(ckv_src, kpe_src, kv_dtype)
    if poison:
        _poison(ckv, kpe, kv_scale, kv_dtype, indptr, indices, last, P, pages)
    return MlaInputs(B, H, P, int(kv_dtype), lengths, q_nope, q_pe, ckv, kpe, kv_scale,
                     indptr, indices, last, float(sm_scale), ckv_src, kpe_src, int(qo_len))


def _poison(ckv, kpe, kv_scale, kv_dtype, indptr, indices, last, P, pages):
    used = np.zeros(pages, bool)
    used[indices] = True
    slot_dead = np.zeros((pages, P), bool)
    slot_dead[~used] = True
    for b in range(indptr.size - 1):
        if indptr[b + 1] > indptr[b]:
            lp = int(indices[indptr[b + 1] - 1])
            slot_dead[lp, int(last[b]):] = True
    if kv_dtype in (KV_BF16, KV_FP16):
        nan = BF16_NAN if kv_dtype == KV_BF16 else FP16_NAN
        ckv[slot_dead] = nan
        kpe[slot_dead] = nan
        return
    kv_scale[slot_dead] = np.nan
    if kv_dtype in (KV_FP8_E4M3, KV_FP8_KPE16):
        ckv[slot_dead] = FP8_E4M3_NAN
    if kv_dtype == KV_FP8_E4M3:
        kpe[slot_dead] = FP8_E4M3_NAN
    if kv_dtype in (KV_FP8_KPE16, KV_INT8_KPE16):
        kpe[slot_dead] = BF16_NAN


# Named workloads (sizes as the pages' regimes: a tiny correctness case, the
# memory-bound h_q = 16 and compute-bound h_q = 128 regimes of FlashMLA PR 233,
# the batch-768 / 64-head case of flashinfer PR 844 with variable lengths, and
# the 8-bit cache).
WORKLOADS = {
    "tiny_b4_h16_l256_p16": dict(batch=4, heads=16, kv_len=256, page=16, kv_dtype=KV_BF16, seed=1),
    "mem_b64_h16_l4096_p64": dict(batch=64, heads=16, kv_len=4096, page=64, kv_dtype=KV_BF16,
                                  seed=2),
    # the memory-bound shape with the other page sizes of the same page
    "mem_b64_h16_l4096_p32": dict(batch=64, heads=16, kv_len=4096, page=32, kv_dtype=KV_BF16,
                                  seed=2),
    "mem_b64_h16_l4096_p16": dict(batch=64, heads=16, kv_len=4096, page=16, kv_dtype=KV_BF16,
                                  seed=2),
    "compute_b64_h128_l4096_p64": dict(batch=64, heads=128, kv_len=4096, page=64,
                                       kv_dtype=KV_BF16, seed=3),
    "varlen_b768_h64_l1to2048_p16": dict(batch=768, heads=64, kv_len=(1, 2048), page=16,
                                         kv_dtype=KV_BF16, seed=4),
    "fp8_b64_h16_l8192_p64": dict(batch=64, heads=16, kv_len=8192, page=64,
                                  kv_dtype=KV_FP8_E4M3, seed=5),
    "fp8_b64_h128_l8192_p64": dict(batch=64, heads=128, kv_len=8192, page=64,
                                   kv_dtype=KV_FP8_E4M3, seed=5),
    "int8_b64_h16_l8192_p64": dict(batch=64, heads=16, kv_len=8192, page=64, kv_dtype=KV_INT8,
                                   seed=5),
    "int8_b64_h128_l8192_p64": dict(batch=64, heads=128, kv_len=8192, page=64, kv_dtype=KV_INT8,
                                    seed=5),
    # the 644-byte record (8-bit ckv, bf16 kpe, fp32 scale on ckv)
    "fp8ckv_bf16kpe_b64_h16_l8192_p64": dict(batch=64, heads=16, kv_len=8192, page=64,
                                             kv_dtype=KV_FP8_KPE16, seed=5),
    "fp8ckv_bf16kpe_b64_h128_l8192_p64": dict(batch=64, heads=128, kv_len=8192, page=64,
                                              kv_dtype=KV_FP8_KPE16, seed=5),
    "int8ckv_bf16kpe_b64_h16_l8192_p64": dict(batch=64, heads=16, kv_len=8192, page=64,
                                              kv_dtype=KV_INT8_KPE16, seed=5),
    "int8ckv_bf16kpe_b64_h128_l8192_p64": dict(batch=64, heads=128, kv_len=8192, page=64,
                                               kv_dtype=KV_INT8_KPE16, seed=5),
    # fp16 inputs (cache, queries and output)
    "fp16_b64_h16_l4096_p64": dict(batch=64, heads=16, kv_len=4096, page=64, kv_dtype=KV_FP16,
                                   seed=2),
    "fp16_b64_h128_l4096_p64": dict(batch=64, heads=128, kv_len=4096, page=64,
                                    kv_dtype=KV_FP16, seed=3),
    # two queries per request (one speculative / next-token-prediction token)
    "mtp_b64_h16_q2_l4096_p64": dict(batch=64, heads=16, kv_len=4096, page=64, kv_dtype=KV_BF16,
                                     seed=6, qo_len=2),
    "mtp_b64_h128_q2_l4096_p64": dict(batch=64, heads=128, kv_len=4096, page=64,
                                      kv_dtype=KV_BF16, seed=6, qo_len=2),
    # long contexts at small batch: every request is cut into many chunks
    # (64 to 256), whose partials a merge spread over the GPU combines
    "longctx_b4_h16_l32768_p64": dict(batch=4, heads=16, kv_len=32768, page=64,
                                      kv_dtype=KV_BF16, seed=7),
    "longctx_b1_h16_l131072_p64": dict(batch=1, heads=16, kv_len=131072, page=64,
                                       kv_dtype=KV_BF16, seed=7),
    "longctx_b16_h64_l8192_p64": dict(batch=16, heads=64, kv_len=8192, page=64,
                                      kv_dtype=KV_BF16, seed=7),
    "longctx_b4_h128_l32768_p64": dict(batch=4, heads=128, kv_len=32768, page=64,
                                       kv_dtype=KV_BF16, seed=7),
}


def workload_lengths(name: str) -> np.ndarray:
    w = WORKLOADS[name]
    if isinstance(w["kv_len"], tuple):
        lo, hi = w["kv_len"]
        rng = _rngs(w["seed"] + 1000, 1)[0]
        return rng.integers(lo, hi + 1, size=w["batch"]).astype(np.int64)
    return np.full(w["batch"], w["kv_len"], np.int64)


def make_workload(name: str, poison: bool = False) -> MlaInputs:
    w = WORKLOADS[name]
    return make_inputs(workload_lengths(name), w["heads"], w["page"], w["kv_dtype"], w["seed"],
                       poison=poison, qo_len=w.get("qo_len", 1))
