"""Python binding of the gfx950 fused exact-attention library (``libfa.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fa.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["FAError", "Params", "Problem", "load", "fwd", "bwd", "bwd_workspace_bytes",
           "dropout_mask", "F32", "BF16", "F16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_EINVAL, FA_EUNSUPPORTED, FA_EHIP = 0, 1, 2, 3
F32, BF16, F16, FP8_E4M3 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class FAError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__("fa status %d: %s" % (status, message))
        self.status = status


class Params(ctypes.Structure):
    """Mirror of ``fa_params_t`` (64 bytes)."""
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dropout_p", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("out_f32", ctypes.c_int32),
                ("Nk", ctypes.c_int32)]


assert ctypes.sizeof(Params) == 64

_lib = None


def load():
    """Load ``libfa.so`` once; raise if it is absent (build it with
    ``python io_aware_exact_20_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfa.so not found at %s: build the HIP library first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, P, sz = ctypes.c_void_p, ctypes.POINTER(Params), ctypes.c_size_t
    lib.fa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_fwd_splitkv.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int32, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [P]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_prepare.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd_prepare.restype = ctypes.c_int
    lib.fa_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd_dkdv.restype = ctypes.c_int
    lib.fa_bwd_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd_dq.restype = ctypes.c_int
    lib.fa_dropout_mask.argtypes = [P, ctypes.c_int64, ctypes.c_int64, vp, vp]
    lib.fa_dropout_mask.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fa_bwd_noalloc.restype = ctypes.c_int
    lib.fa_bwd_noalloc_max_workspace_bytes.argtypes = []
    lib.fa_bwd_noalloc_max_workspace_bytes.restype = sz
    lib.fa_unit_order.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, vp, vp]
    lib.fa_unit_order.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != FA_OK:
        msg = _lib.fa_last_error().decode() or _lib.fa_status_str(status).decode()
        raise FAError(status, msg)


def make_params(B, H, N, d, dtype=BF16, scale=None, causal=False, dropout_p=0.0, seed=0,
                out_f32=False, Nk=0) -> Params:
    return Params(B=B, H=H, N=N, d=d, dtype=dtype,
                  causal=int(bool(causal)),
                  scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
                  dropout_p=float(dropout_p), seed=int(seed) & (2**64 - 1),
                  out_f32=int(bool(out_f32)), Nk=int(Nk))


def _params_for(q: torch.Tensor, scale, causal, dropout_p, seed, out_f32) -> Params:
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("unsupported dtype %s" % q.dtype)
    B, H, N, d = q.shape
    return make_params(B, H, N, d, _DTYPE_CODE[q.dtype], scale, causal, dropout_p, seed,
                       out_f32)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, like, name, dtype=None, shape=None):
    shape = tuple(like.shape) if shape is None else tuple(shape)
    if not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
        raise ValueError("%s must be a contiguous device tensor of shape %s" % (name, shape))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s (got %s)" % (name, dtype, t.dtype))
    if t.device != like.device:
        raise ValueError("%s must be on %s (got %s)" % (name, like.device, t.device))


def _check_bwd_inputs(q, o, lse, dout, out_f32):
    """o in the forward's output type, lse float32 [B,H,N], dout in q's type."""
    _need(o, q, "o", dtype=torch.float32 if out_f32 else q.dtype)
    _need(lse, q, "lse", dtype=torch.float32, shape=q.shape[:3])
    _need(dout, q, "dout", dtype=q.dtype)


def _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32):
    """Checks q [B,H,N,d] and k, v [B,H,Nk,d]; the params (Nk set when != N)."""
    _need(q, q, "q")
    _need(k, k, "k")
    _need(v, k, "v")
    if k.dim() != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("k, v must be [B, H, Nk, d] with q's B, H, d")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    p = _params_for(q, scale, causal, dropout_p, seed, out_f32)
    if k.shape[2] != q.shape[2]:
        p.Nk = k.shape[2]
    return p


def fwd(q, k, v, scale=None, causal=False, dropout_p=0.0, seed=0, out_f32=False):
    """Fused forward: returns (o [B,H,N,d], lse [B,H,N] float32); k and v
    may hold Nk != N keys (see ``fa_params_t.Nk``)."""
    lib = load()
    p = _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32)
    o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                      _stream(q)))
    return o, lse


def fwd_fp8(q, k, v, descale_q, descale_k, descale_v, scale=None, causal=False,
            out_f32=False):
    """Forward with OCP e4m3 inputs (``fa_fwd_fp8``): q [B,H,N,128], k, v
    [B,H,Nk,128] as torch.float8_e4m3fn device tensors, descale_* float32
    [B,H] device tensors (the inputs are q * descale_q[b, h], ...).  Returns
    (o bfloat16 or float32 [B,H,N,128], lse float32 [B,H,N])."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError("%s must be torch.float8_e4m3fn (got %s)" % (n, t.dtype))
    _need(q, q, "q")
    _need(k, k, "k")
    _need(v, k, "v")
    if k.dim() != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("k, v must be [B, H, Nk, d] with q's B, H, d")
    B, H, N, d = q.shape
    for t, n in ((descale_q, "descale_q"), (descale_k, "descale_k"), (descale_v, "descale_v")):
        _need(t, q, n, dtype=torch.float32, shape=(B, H))
    p = make_params(B, H, N, d, FP8_E4M3, scale, causal, 0.0, 0, out_f32,
                    k.shape[2] if k.shape[2] != N else 0)
    o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_fp8(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(descale_q),
                          _ptr(descale_k), _ptr(descale_v), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


def fwd_splitkv(q, k, v, num_splits, scale=None, causal=False, dropout_p=0.0, seed=0,
                out_f32=False, workspace=None):
    """Forward with the keys split into up to ``num_splits`` chunks and
    merged (``fa_fwd_splitkv``); same results as ``fwd``."""
    lib = load()
    p = _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32)
    need = lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), int(num_splits))
    if need == ctypes.c_size_t(-1).value:
        raise FAError(FA_EINVAL, lib.fa_last_error().decode())
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_splitkv(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              int(num_splits), _ptr(workspace), workspace.numel(), _stream(q)))
    return o, lse


def bwd_workspace_bytes(q, scale=None, causal=False, dropout_p=0.0, seed=0, out_f32=False):
    lib = load()
    p = _params_for(q, scale, causal, dropout_p, seed, out_f32)
    n = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    if n == ctypes.c_size_t(-1).value:
        raise FAError(FA_EINVAL, lib.fa_last_error().decode())
    return n


def bwd(q, k, v, o, lse, dout, scale=None, causal=False, dropout_p=0.0, seed=0,
        out_f32=False, workspace=None):
    """Fused backward: returns (dq, dk, dv) with the forward's output type
    (k, v and so dk, dv may hold Nk != N keys)."""
    lib = load()
    p = _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32)
    _check_bwd_inputs(q, o, lse, dout, out_f32)
    out_dtype = torch.float32 if out_f32 else q.dtype
    dq = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    dk = torch.empty(k.shape, dtype=out_dtype, device=q.device)
    dv = torch.empty(k.shape, dtype=out_dtype, device=q.device)
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.fa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                      _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                      workspace.numel(), _stream(q)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, scale=None, causal=False, dropout_p=0.0, seed=0,
                out_f32=False, out=None):
    """``fa_bwd_noalloc``: the backward with the library's static scratch in
    place of a workspace.  ``out`` = (dq, dk, dv) preallocated by the caller
    (allocated here when None)."""
    lib = load()
    p = _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32)
    _check_bwd_inputs(q, o, lse, dout, out_f32)
    out_dtype = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = (torch.empty(q.shape, dtype=out_dtype, device=q.device),
               torch.empty(k.shape, dtype=out_dtype, device=q.device),
               torch.empty(k.shape, dtype=out_dtype, device=q.device))
    dq, dk, dv = out
    _need(dq, q, "dq", dtype=out_dtype)
    _need(dk, k, "dk", dtype=out_dtype)
    _need(dv, k, "dv", dtype=out_dtype)
    _check(lib.fa_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(q)))
    return dq, dk, dv


class Problem:
    """Preallocated outputs and workspace for repeated calls on one shape
    (the benchmark's launch configuration).  Each method enqueues exactly
    one library call on the current stream."""

    def __init__(self, q, k, v, dout=None, scale=None, causal=False, dropout_p=0.0, seed=0,
                 out_f32=False):
        lib = load()
        self.q, self.k, self.v, self.dout = q, k, v, dout
        self.p = _fwd_params(q, k, v, scale, causal, dropout_p, seed, out_f32)
        odt = torch.float32 if out_f32 else q.dtype
        self.o = torch.empty(q.shape, dtype=odt, device=q.device)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        if dout is not None:
            _need(dout, q, "dout", dtype=q.dtype)
            self.dq = torch.empty(q.shape, dtype=odt, device=q.device)
            self.dk = torch.empty(k.shape, dtype=odt, device=q.device)
            self.dv = torch.empty(k.shape, dtype=odt, device=q.device)
            n = lib.fa_bwd_workspace_bytes(ctypes.byref(self.p))
            self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
        self._s = _stream(q)

    def fwd(self):
        _check(_lib.fa_fwd(ctypes.byref(self.p), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                           _ptr(self.o), _ptr(self.lse), self._s))

    def bwd_prepare(self):
        _check(_lib.fa_bwd_prepare(ctypes.byref(self.p), _ptr(self.o), _ptr(self.lse),
                                   _ptr(self.dout), _ptr(self.ws), self.ws.numel(), self._s))

    def bwd_dkdv(self):
        _check(_lib.fa_bwd_dkdv(ctypes.byref(self.p), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                                _ptr(self.lse), _ptr(self.dout), _ptr(self.dk), _ptr(self.dv),
                                _ptr(self.ws), self.ws.numel(), self._s))

    def bwd_dq(self):
        _check(_lib.fa_bwd_dq(ctypes.byref(self.p), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                              _ptr(self.lse), _ptr(self.dout), _ptr(self.dq), _ptr(self.ws),
                              self.ws.numel(), self._s))

    def bwd(self):
        self.bwd_prepare()
        self.bwd_dkdv()
        self.bwd_dq()


def unit_order(BH, nb, group):
    """(bh, rank) uint32 arrays of the kernels' work-unit order for BH heads
    of nb blocks each and heads grouped by ``group`` (host only)."""
    import numpy as np
    lib = load()
    bh = np.empty(BH * nb, dtype=np.uint32)
    rank = np.empty(BH * nb, dtype=np.uint32)
    _check(lib.fa_unit_order(BH, nb, group, bh.ctypes.data, rank.ctypes.data))
    return bh, rank


def dropout_mask(B, H, N, dropout_p, seed, b, h, device="cuda"):
    """Keep mask (uint8 [N, N], 1 = kept) of plane (b, h) from the device generator."""
    lib = load()
    p = make_params(B, H, N, 64, BF16, None, False, dropout_p, seed, False)
    m = torch.empty((N, N), dtype=torch.uint8, device=device)
    _check(lib.fa_dropout_mask(ctypes.byref(p), b, h, _ptr(m),
                               ctypes.c_void_p(torch.cuda.current_stream(m.device).cuda_stream)))
    return m
