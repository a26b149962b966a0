"""Paged MLA decode (absorbed-MQA form) for MI355X / gfx950.

Thin ctypes binding over the C ABI in ``include/mla_decode.h``
(``libmla_decode.so``, built in-tree by ``mla_paged_kv_decode_amd.build``).
This module only marshals arguments: every step of the decode runs in the HIP
kernels of the library.  PyTorch supplies device memory and streams.  There is
no CPU fallback: if the library is missing, every call raises.

Names follow the pages' notation: q_nope [B, H, 512], q_pe [B, H, 64],
ckv [pages, P, 512], kpe [pages, P, 64], kv_indptr / kv_indices /
kv_last_page_len (the paged KV table), sm_scale, o [B, H, 512] and lse [B, H].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_OK = 0
KV_BF16, KV_FP8_E4M3, KV_INT8 = 0, 1, 2
# the 644-byte record: 8-bit ckv codes, bf16 kpe, fp32 scale on ckv only
KV_FP8_E4M3_KPE_BF16, KV_INT8_KPE_BF16 = 3, 4
_KPE_BF16 = (KV_FP8_E4M3_KPE_BF16, KV_INT8_KPE_BF16)
# fp16 inputs: fp16 cache, queries and output
KV_FP16 = 5
D_CKV, D_KPE = 512, 64
# MLA_NOALLOC_SCRATCH_BYTES: the per-GPU array that mla_decode_run_noalloc uses
NOALLOC_SCRATCH_BYTES = 72 << 20

EXPORTED_SYMBOLS = (
    "mla_decode_workspace_bytes",
    "mla_decode_plan",
    "mla_decode_run",
    "mla_decode_run_noalloc",
    "mla_decode_plan_destroy",
    "mla_status_string",
    "mla_last_error",
    "mla_decode_plan_info",
    "mla_decode_plan_segments",
    "mla_decode_plan_set_events",
    "mla_cache_append",
    "mla_peak_stream_read",
    "mla_peak_mfma_bf16",
)

_lib = None


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        msg = lib.mla_status_string(status).decode()
        detail = lib.mla_last_error().decode()
        super().__init__("%s: %s (status %d)%s" % (what, msg, status,
                                                   (" - " + detail) if detail else ""))
        self.status = status


class PlanOpts(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("force_splits", ctypes.c_int32),
                ("max_workers", ctypes.c_int32), ("head_split", ctypes.c_int32),
                ("qo_len", ctypes.c_int32), ("l2_domains", ctypes.c_int32)]


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmla_decode.so is not built (%s); run "
                           "`python -m mla_paged_kv_decode_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mla_decode_workspace_bytes.argtypes = [i32, i32, ctypes.POINTER(PlanOpts)]
    lib.mla_decode_workspace_bytes.restype = sz
    lib.mla_decode_plan.argtypes = [ctypes.POINTER(P), P, P, i32, i32, i32, i32,
                                    ctypes.POINTER(PlanOpts), P, sz, P]
    lib.mla_decode_plan.restype = ctypes.c_int
    lib.mla_decode_run.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.mla_decode_run.restype = ctypes.c_int
    lib.mla_decode_run_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.mla_decode_run_noalloc.restype = ctypes.c_int
    lib.mla_decode_plan_destroy.argtypes = [P]
    lib.mla_decode_plan_destroy.restype = None
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_decode_plan_info.argtypes = [P, P]
    lib.mla_decode_plan_info.restype = ctypes.c_int
    lib.mla_decode_plan_segments.argtypes = [P, P, P]
    lib.mla_decode_plan_segments.restype = ctypes.c_int
    lib.mla_decode_plan_set_events.argtypes = [P, P, P]
    lib.mla_decode_plan_set_events.restype = ctypes.c_int
    lib.mla_cache_append.argtypes = [P, P, P, i32, i32, P, P, P, P]
    lib.mla_cache_append.restype = ctypes.c_int
    lib.mla_peak_stream_read.argtypes = [P, sz, P, i32, ctypes.POINTER(ctypes.c_float), P]
    lib.mla_peak_stream_read.restype = ctypes.c_int
    lib.mla_peak_mfma_bf16.argtypes = [P, i32, ctypes.POINTER(ctypes.c_float), P]
    lib.mla_peak_mfma_bf16.restype = ctypes.c_int
    _lib = lib
    return lib


def _opts(num_cus=0, force_splits=0, max_workers=0, head_split=0, qo_len=1,
          l2_domains=0) -> PlanOpts:
    return PlanOpts(int(num_cus), int(force_splits), int(max_workers), int(head_split),
                    int(qo_len), int(l2_domains))


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(batch: int, num_heads: int, num_cus: int = 0, force_splits: int = 0,
                    max_workers: int = 0, head_split: int = 0, qo_len: int = 1) -> int:
    o = _opts(num_cus, force_splits, max_workers, head_split, qo_len)
    n = load_library().mla_decode_workspace_bytes(int(batch), int(num_heads), ctypes.byref(o))
    if n == 0:
        raise MlaError(-2, "mla_decode_workspace_bytes")
    return int(n)


class Plan:
    """A split-KV schedule for one batch (``mla_decode_plan``).

    ``workspace`` is a device uint8 tensor of at least ``workspace_bytes``;
    ``None`` makes a host-only plan that can be inspected but not run.
    ``qo_len`` queries per request: q and o are [batch * qo_len, H, ...], with
    the causal mask aligned to the end of each request.
    """

    def __init__(self, kv_indptr, kv_last_page_len, num_heads: int, page_size: int,
                 kv_dtype: int = KV_BF16, workspace=None, num_cus: int = 0,
                 force_splits: int = 0, max_workers: int = 0, head_split: int = 0,
                 stream=None, qo_len: int = 1, l2_domains: int = 0):
        lib = load_library()
        self._lib = lib
        ip = _host_i32(kv_indptr)
        lp = _host_i32(kv_last_page_len)
        self.batch = int(ip.size - 1)
        self.num_pages_used = int(ip[-1]) if ip.size else 0  # kv_indices entries the plan reads
        self.num_heads = int(num_heads)
        self.page_size = int(page_size)
        self.kv_dtype = int(kv_dtype)
        self.qo_len = int(qo_len)
        self.workspace = workspace
        o = _opts(num_cus, force_splits, max_workers, head_split, qo_len, l2_domains)
        h = ctypes.c_void_p()
        ws_ptr, ws_n, sp = None, 0, None
        if workspace is not None:
            ws_ptr = _dptr(workspace)
            ws_n = workspace.numel() * workspace.element_size()
            sp = _stream_ptr(stream)
        st = lib.mla_decode_plan(ctypes.byref(h), ip.ctypes.data_as(ctypes.c_void_p),
                                 lp.ctypes.data_as(ctypes.c_void_p), self.batch, self.num_heads,
                                 self.page_size, self.kv_dtype, ctypes.byref(o), ws_ptr, ws_n, sp)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_plan")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.mla_decode_plan_destroy(h)
            self._h = None

    def info(self) -> dict:
        buf = np.zeros(16, np.int32)
        st = self._lib.mla_decode_plan_info(self._h, buf.ctypes.data_as(ctypes.c_void_p))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_plan_info")
        keys = ("batch", "num_heads", "page_size", "kv_dtype", "num_workers", "num_segments",
                "num_partials", "num_split_requests", "granularity", "waves", "head_split",
                "kernel_heads", "qo_len", "one_seg", "req_div", "req_deal")
        return {k: int(v) for k, v in zip(keys, buf)}

    def segments(self):
        inf = self.info()
        seg = np.zeros((max(1, inf["num_segments"]), 4), np.int32)
        wp = np.zeros(inf["num_workers"] + 1, np.int32)
        st = self._lib.mla_decode_plan_segments(self._h, seg.ctypes.data_as(ctypes.c_void_p),
                                                wp.ctypes.data_as(ctypes.c_void_p))
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_plan_segments")
        return seg[:inf["num_segments"]], wp

    def set_events(self, before, after) -> None:
        """Raw hipEvent_t handles (ints) that run() fills with the start and the
        end of the decode kernel alone, from its own dispatch (the merge launch of
        split requests is not included)."""
        st = self._lib.mla_decode_plan_set_events(self._h, before, after)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode_plan_set_events")

    def run(self, q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr, kv_indices, kv_last_page_len,
            sm_scale: float, o, lse, stream=None) -> None:
        """``mla_decode_run`` on device tensors (o and lse are written)."""
        self._run(self._lib.mla_decode_run, "mla_decode_run", q_nope, q_pe, ckv, kpe, kv_scale,
                  kv_indptr, kv_indices, kv_last_page_len, sm_scale, o, lse, stream)

    def run_noalloc(self, q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr, kv_indices,
                    kv_last_page_len, sm_scale: float, o, lse, stream=None) -> None:
        """``mla_decode_run_noalloc``: as ``run``, with the work list and partials in
        the library's per-GPU scratch instead of the plan's workspace (which may be
        None).  Calls that overlap on one GPU race."""
        self._run(self._lib.mla_decode_run_noalloc, "mla_decode_run_noalloc", q_nope, q_pe, ckv,
                  kpe, kv_scale, kv_indptr, kv_indices, kv_last_page_len, sm_scale, o, lse,
                  stream)

    def _run(self, fn, name, q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr, kv_indices,
             kv_last_page_len, sm_scale, o, lse, stream) -> None:
        import torch
        B, H = self.batch * self.qo_len, self.num_heads
        t16 = torch.float16 if self.kv_dtype == KV_FP16 else torch.bfloat16
        if q_nope.dtype != t16 or q_pe.dtype != t16:
            raise ValueError("q_nope / q_pe must be %s" % t16)
        if tuple(q_nope.shape) != (B, H, D_CKV) or tuple(q_pe.shape) != (B, H, D_KPE):
            raise ValueError("q_nope / q_pe shape mismatch with the plan")
        if tuple(o.shape) != (B, H, D_CKV) or o.dtype != t16:
            raise ValueError("o must be %s [B * qo_len, H, 512]" % t16)
        if tuple(lse.shape) != (B, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B * qo_len, H]")
        for name, t in (("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
                        ("kv_last_page_len", kv_last_page_len)):
            if t.dtype != torch.int32:
                raise ValueError(name + " must be int32")
        # the device page table is the plan's batch, as planned or grown since
        # (the kernels read it without bounds checks)
        if kv_indptr.numel() != self.batch + 1 or kv_last_page_len.numel() != self.batch:
            raise ValueError("kv_indptr / kv_last_page_len sizes differ from the plan's")
        if kv_indices.numel() < self.num_pages_used:
            raise ValueError("kv_indices holds fewer entries than the plan-time kv_indptr[-1]")
        if ckv.dim() != 3 or ckv.shape[1] != self.page_size or ckv.shape[2] != D_CKV:
            raise ValueError("ckv must be [pages, page_size, 512]")
        if kpe.dim() != 3 or kpe.shape[1] != self.page_size or kpe.shape[2] != D_KPE:
            raise ValueError("kpe must be [pages, page_size, 64]")
        if self.kv_dtype in (KV_BF16, KV_FP16):
            if ckv.dtype != t16 or kpe.dtype != t16:
                raise ValueError("%s cache expected" % t16)
            if kv_scale is not None:
                raise ValueError("kv_scale must be None for a 16-bit cache")
        else:
            codes = (torch.uint8, torch.float8_e4m3fn) \
                if self.kv_dtype in (KV_FP8_E4M3, KV_FP8_E4M3_KPE_BF16) else (torch.uint8, torch.int8)
            kpe_ok = kpe.dtype == torch.bfloat16 if self.kv_dtype in _KPE_BF16 else kpe.dtype in codes
            if ckv.dtype not in codes or not kpe_ok:
                raise ValueError("8-bit cache expected (one byte per ckv value; kpe one byte, "
                                 "or bf16 for the 644-byte layouts)")
            if (kv_scale is None or kv_scale.dtype != torch.float32
                    or tuple(kv_scale.shape) != tuple(ckv.shape[:2])):
                raise ValueError("kv_scale must be float32 [pages, page_size]")
        if kpe.shape[0] != ckv.shape[0]:
            raise ValueError("ckv and kpe must hold the same pages")
        for name, t in (("q_nope", q_nope), ("q_pe", q_pe), ("ckv", ckv), ("kpe", kpe),
                        ("kv_scale", kv_scale), ("o", o), ("lse", lse)):
            if t is not None and not t.is_contiguous():
                raise ValueError(name + " must be contiguous")
        st = fn(self._h, _dptr(q_nope), _dptr(q_pe), _dptr(ckv), _dptr(kpe), _dptr(kv_scale),
                _dptr(kv_indptr), _dptr(kv_indices), _dptr(kv_last_page_len), float(sm_scale),
                _dptr(o), _dptr(lse), _stream_ptr(stream))
        if st != MLA_OK:
            raise MlaError(st, name)


def cache_append(ckv_new, kpe_new, slots, ckv, kpe, kv_dtype: int = KV_BF16, kv_scale=None,
                 stream=None) -> None:
    """``mla_cache_append``: write new tokens (bf16 ckv_new [n, 512], kpe_new
    [n, 64]) into cache rows ``slots`` (int64 [n], page * page_size + position;
    negative = skip), quantising them for an 8-bit cache."""
    import torch
    n = int(ckv_new.shape[0])
    t16 = torch.float16 if kv_dtype == KV_FP16 else torch.bfloat16
    if ckv_new.dtype != t16 or kpe_new.dtype != t16:
        raise ValueError("new tokens must be %s" % t16)
    if tuple(ckv_new.shape) != (n, D_CKV) or tuple(kpe_new.shape) != (n, D_KPE):
        raise ValueError("ckv_new must be [n, 512] and kpe_new [n, 64]")
    if slots.dtype != torch.int64 or tuple(slots.shape) != (n,):
        raise ValueError("slots must be int64 [n]")
    if ckv.dim() != 3 or ckv.shape[2] != D_CKV or kpe.dim() != 3 or kpe.shape[2] != D_KPE \
            or tuple(ckv.shape[:2]) != tuple(kpe.shape[:2]):
        raise ValueError("ckv / kpe must be [pages, page_size, 512 / 64]")
    if kv_dtype in (KV_BF16, KV_FP16):
        if ckv.dtype != t16 or kpe.dtype != t16 or kv_scale is not None:
            raise ValueError("%s cache expected, without kv_scale" % t16)
    else:
        kpe_size = 2 if kv_dtype in _KPE_BF16 else 1
        if ckv.element_size() != 1 or kpe.element_size() != kpe_size:
            raise ValueError("8-bit cache expected (bf16 kpe for the 644-byte layouts)")
        if kv_scale is None or kv_scale.dtype != torch.float32 \
                or tuple(kv_scale.shape) != tuple(ckv.shape[:2]):
            raise ValueError("kv_scale must be float32 [pages, page_size]")
    st = load_library().mla_cache_append(_dptr(ckv_new), _dptr(kpe_new), _dptr(slots), n,
                                         int(kv_dtype), _dptr(ckv), _dptr(kpe), _dptr(kv_scale),
                                         _stream_ptr(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_cache_append")


def peak_stream_read_gbs(nbytes: int = 4 << 30, iters: int = 20, stream=None) -> float:
    """Measured HBM read bandwidth (GB/s): median pass of a 16-byte-load read
    over a fresh device buffer of nbytes."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    ms = ctypes.c_float()
    st = load_library().mla_peak_stream_read(_dptr(buf), nbytes, _dptr(sink), int(iters),
                                             ctypes.byref(ms), _stream_ptr(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_peak_stream_read")
    return nbytes / (ms.value * 1e-3) / 1e9


def peak_mfma_bf16_tflops(iters: int = 10, stream=None) -> float:
    """Measured dense bf16 MFMA throughput (TFLOP/s)."""
    import torch
    sink = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    tf = ctypes.c_float()
    st = load_library().mla_peak_mfma_bf16(_dptr(sink), int(iters), ctypes.byref(tf),
                                           _stream_ptr(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_peak_mfma_bf16")
    return float(tf.value)


def decode(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_last_page_len, sm_scale: float,
           kv_dtype: int = KV_BF16, kv_scale=None, kv_indptr_host=None,
           kv_last_page_len_host=None, force_splits: int = 0, head_split: int = 0,
           stream=None, qo_len: int = 1):
    """One-shot plan + run.  Returns (o, lse) as new device tensors."""
    import torch
    NQ, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    B = int(kv_indptr.shape[0]) - 1
    if NQ != B * qo_len:
        raise ValueError("q_nope must hold batch * qo_len query rows")
    P = int(ckv.shape[1])
    ip_h = kv_indptr if kv_indptr_host is None else kv_indptr_host
    lp_h = kv_last_page_len if kv_last_page_len_host is None else kv_last_page_len_host
    ws = torch.empty(workspace_bytes(B, H, force_splits=force_splits, head_split=head_split,
                                     qo_len=qo_len),
                     dtype=torch.uint8, device=q_nope.device)
    plan = Plan(ip_h, lp_h, H, P, kv_dtype, ws, force_splits=force_splits, head_split=head_split,
                stream=stream, qo_len=qo_len)
    o = torch.empty((NQ, H, D_CKV), dtype=q_nope.dtype, device=q_nope.device)
    lse = torch.empty((NQ, H), dtype=torch.float32, device=q_nope.device)
    plan.run(q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr, kv_indices, kv_last_page_len, sm_scale,
             o, lse, stream)
    return o, lse
