"""fp64 CPU oracle for paged MLA decode (absorbed-MQA form).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU path
(``mla_paged_kv_decode_amd``) never imports it, and the two share no code:
the oracle is plain C (``mla_oracle.c``), compiled with gcc, with its own
bf16 / e4m3fn / int8 decoders.

What it computes is stated in the header of ``mla_oracle.c``; in short, for
request b and head h over the request's kv_len tokens gathered through the
page table: s_t = sm_scale * (q_nope . ckv_t + q_pe . kpe_t),
O = softmax(s) . ckv (512 wide), LSE = ln sum_t exp(s_t).  Sources: the
"Benchmarking MLA" page (flashinfer issue 700; the absorbed form with
qk dim 512 + 64 and v dim 512, ckv used as both key and value, and the
nvbench argument list), and FlashMLA PR 233 "What is added" (paged cache,
8-bit cache with one scale per token, deterministic split combine).

Every function here is pinned by ``tests/test_oracle_pins.py`` against brute
force, closed forms, invariants and library routines; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

KV_BF16, KV_FP8_E4M3, KV_INT8 = 0, 1, 2
# 644-byte record: 8-bit ckv codes, bf16 kpe, fp32 scale on ckv only
KV_FP8_KPE16, KV_INT8_KPE16 = 3, 4
# fp16 cache, with fp16 queries
KV_FP16 = 5
D_CKV, D_KPE = 512, 64

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libmla_oracle.so``."""
    global _lib
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_dec_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_bf16.restype = f64
    lib.oracle_dec_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e4m3fn.restype = f64
    lib.oracle_dec_int8.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_int8.restype = f64
    lib.oracle_dec_fp16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_fp16.restype = f64
    lib.oracle_kv_len.argtypes = [P, P, i32, i32]
    lib.oracle_kv_len.restype = i64
    lib.mla_oracle_decode.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f64, P, i64,
                                      P, P, i32]
    lib.mla_oracle_decode.restype = ctypes.c_int
    lib.mla_oracle_partial.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, f64, i32, i32,
                                       i32, i64, i64, P, P]
    lib.mla_oracle_partial.restype = ctypes.c_int
    lib.mla_oracle_combine.argtypes = [i32, P, P, P, P]
    lib.mla_oracle_combine.restype = None
    lib.mla_oracle_quantize.argtypes = [i32, i32, P, P, P, P, P]
    lib.mla_oracle_quantize.restype = ctypes.c_int
    lib.oracle_enc_e4m3fn.argtypes = [ctypes.c_float]
    lib.oracle_enc_e4m3fn.restype = ctypes.c_uint8
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def dec_bf16(bits: int) -> float:
    return _load().oracle_dec_bf16(int(bits) & 0xFFFF)


def dec_e4m3fn(code: int) -> float:
    return _load().oracle_dec_e4m3fn(int(code) & 0xFF)


def dec_fp16(bits: int) -> float:
    return _load().oracle_dec_fp16(int(bits))


def dec_int8(code: int) -> float:
    return _load().oracle_dec_int8(int(code) & 0xFF)


def kv_len(kv_indptr, kv_last_page_len, page_size: int, b: int) -> int:
    ip = _c(kv_indptr, np.int32)
    lp = _c(kv_last_page_len, np.int32)
    return int(_load().oracle_kv_len(_ptr(ip), _ptr(lp), int(page_size), int(b)))


def _kv_arrays(kv_dtype, ckv, kpe):
    if kv_dtype in (KV_BF16, KV_FP16):
        return _c(ckv, np.uint16), _c(kpe, np.uint16)
    if kv_dtype in (KV_FP8_KPE16, KV_INT8_KPE16):
        return _c(ckv, np.uint8), _c(kpe, np.uint16)
    return _c(ckv, np.uint8), _c(kpe, np.uint8)


def decode(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_last_page_len, sm_scale: float,
           page_size: int, kv_dtype: int = KV_BF16, kv_scale=None, rows=None, threads: int = 0,
           qo_len: int = 1):
    """fp64 decode.  Inputs are host numpy arrays: bf16 tensors as uint16 bit
    patterns (fp16 ones for kv_dtype KV_FP16, queries included), 8-bit caches
    as uint8 codes with an fp32 ``kv_scale[pages, P]``.
    With qo_len > 1 the queries are [B * qo_len, H, *] and query i of request b
    sees its first L_b - (qo_len - 1 - i) tokens (causal, queries at the end).

    Returns (o, lse): o is float64 [B * qo_len, H, 512] (or [len(rows), 512]
    when a list of flattened (b * qo_len + i) * H + h rows is given) and lse
    float64 [B * qo_len, H] (or [len(rows)]).
    """
    qn = _c(q_nope, np.uint16)
    qp = _c(q_pe, np.uint16)
    NQ, H = qn.shape[0], qn.shape[1]
    assert qo_len >= 1 and NQ % qo_len == 0
    B = NQ // qo_len
    assert qn.shape == (NQ, H, D_CKV) and qp.shape == (NQ, H, D_KPE)
    ck, kp = _kv_arrays(kv_dtype, ckv, kpe)
    sc = _c(kv_scale, np.float32)
    ip = _c(kv_indptr, np.int32)
    ix = _c(kv_indices, np.int32)
    lp = _c(kv_last_page_len, np.int32)
    if threads <= 0:
        # the host's cores, capped by OMP_NUM_THREADS when set (the share of a
        # machine this process may use)
        threads = os.cpu_count() or 1
        env = os.environ.get("OMP_NUM_THREADS", "")
        if env.isdigit() and int(env) > 0:
            threads = min(threads, int(env))
    if rows is None:
        o = np.zeros((NQ, H, D_CKV), np.float64)
        lse = np.zeros((NQ, H), np.float64)
        rr, nr = None, 0
    else:
        rr = _c(rows, np.int32)
        nr = rr.size
        o = np.zeros((nr, D_CKV), np.float64)
        lse = np.zeros((nr,), np.float64)
    st = _load().mla_oracle_decode(B, int(qo_len), H, int(page_size), int(kv_dtype), _ptr(qn),
                                    _ptr(qp),
                                    _ptr(ck), _ptr(kp), _ptr(sc), _ptr(ip), _ptr(ix), _ptr(lp),
                                    float(sm_scale), _ptr(rr), nr, _ptr(o), _ptr(lse), int(threads))
    if st != 0:
        raise RuntimeError("mla_oracle_decode failed")
    return o, lse


def partial(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_last_page_len, sm_scale: float,
            page_size: int, b: int, h: int, t0: int, t1: int, kv_dtype: int = KV_BF16,
            kv_scale=None, qo_len: int = 1, qi: int = 0):
    """Partial (O_i [512], LSE_i) of head h of query qi of request b over tokens
    [t0, t1), tokens past the query's causal limit excluded."""
    qn = _c(q_nope, np.uint16)
    qp = _c(q_pe, np.uint16)
    B, H = qn.shape[0] // qo_len, qn.shape[1]
    ck, kp = _kv_arrays(kv_dtype, ckv, kpe)
    sc = _c(kv_scale, np.float32)
    ip = _c(kv_indptr, np.int32)
    ix = _c(kv_indices, np.int32)
    lp = _c(kv_last_page_len, np.int32)
    o = np.zeros((D_CKV,), np.float64)
    lse = np.zeros((1,), np.float64)
    st = _load().mla_oracle_partial(B, int(qo_len), H, int(page_size), int(kv_dtype), _ptr(qn),
                                     _ptr(qp), _ptr(ck), _ptr(kp), _ptr(sc), _ptr(ip), _ptr(ix),
                                     _ptr(lp), float(sm_scale), int(b), int(qi), int(h), int(t0),
                                     int(t1), _ptr(o), _ptr(lse))
    if st != 0:
        raise RuntimeError("mla_oracle_partial: bad range")
    return o, float(lse[0])


def combine(lse_parts, o_parts):
    """Fixed-order merge of split partials: returns (O [512], LSE)."""
    lp = _c(lse_parts, np.float64).reshape(-1)
    op = _c(o_parts, np.float64).reshape(lp.size, D_CKV)
    o = np.zeros((D_CKV,), np.float64)
    lse = np.zeros((1,), np.float64)
    _load().mla_oracle_combine(int(lp.size), _ptr(lp), _ptr(op), _ptr(o), _ptr(lse))
    return o, float(lse[0])


def enc_e4m3fn(v: float) -> int:
    """e4m3fn code of a binary32 value: nearest, ties to even, saturated."""
    return int(_load().oracle_enc_e4m3fn(float(v)))


def quantize(ckv_new: np.ndarray, kpe_new: np.ndarray, kv_dtype: int):
    """Quantise new tokens for an 8-bit cache (see ``mla_oracle_quantize``):
    bf16 bits [n, 512] and [n, 64] -> (ckv codes uint8 [n, 512], kpe codes
    uint8 [n, 64], scales float32 [n]).  For the 644-byte layouts only ckv is
    quantised and the kpe element is the bf16 input, unchanged."""
    ckv_new = np.ascontiguousarray(ckv_new, np.uint16)
    kpe_new = np.ascontiguousarray(kpe_new, np.uint16)
    n = ckv_new.shape[0]
    assert ckv_new.shape == (n, D_CKV) and kpe_new.shape == (n, D_KPE)
    cc = np.zeros((n, D_CKV), np.uint8)
    kc = np.zeros((n, D_KPE), np.uint8)
    sc = np.zeros(n, np.float32)
    P = ctypes.c_void_p
    st = _load().mla_oracle_quantize(n, int(kv_dtype), ckv_new.ctypes.data_as(P),
                                     kpe_new.ctypes.data_as(P), cc.ctypes.data_as(P),
                                     kc.ctypes.data_as(P), sc.ctypes.data_as(P))
    if st != 0:
        raise ValueError("unsupported kv_dtype for quantisation")
    if kv_dtype in (KV_FP8_KPE16, KV_INT8_KPE16):
        return cc, kpe_new.copy(), sc
    return cc, kc, sc
