"""Exact-attention oracle: plain fp64 CPU reference (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library.  The C
source (``oracle.c``) holds the arithmetic; this module only compiles it
with the host compiler and marshals numpy arrays.

Every function takes tensors laid out as [B, H, N, d] (``lse``: [B, H, N])
and evaluates the plain definition of softmax(scale * Q K^T + mask) V in
double precision -- see the header of ``oracle.c`` for the definition, its
source passages and the dropout generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source file into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (host only)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    i64, dbl, vp, i32, u64 = (ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
                              ctypes.c_int, ctypes.c_uint64)
    lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_drop_threshold.argtypes = [dbl]
    lib.oracle_drop_threshold.restype = ctypes.c_uint32
    lib.oracle_keep_scale.argtypes = [dbl]
    lib.oracle_keep_scale.restype = dbl
    lib.oracle_dropout_mask.argtypes = [i64, dbl, u64, i64, i64, vp]
    lib.oracle_dropout_mask.restype = i32
    lib.oracle_fwd_rows.argtypes = [i64, i64, vp, vp, vp, dbl, i32, dbl, u64, i64, i64,
                                    vp, i64, vp, vp]
    lib.oracle_fwd_rows.restype = i32
    lib.oracle_fwd_cross.argtypes = [i64, i64, i64, vp, vp, vp, dbl, i32, dbl, u64, i64, i64,
                                     vp, vp]
    lib.oracle_fwd_cross.restype = i32
    lib.oracle_bwd_cross.argtypes = [i64, i64, i64, vp, vp, vp, vp, dbl, i32, dbl, u64, i64,
                                     i64, vp, vp, vp, vp, vp]
    lib.oracle_bwd_cross.restype = i32
    lib.oracle_probs.argtypes = [i64, i64, vp, vp, dbl, i32, dbl, u64, i64, i64, vp, vp]
    lib.oracle_probs.restype = i32
    lib.oracle_bwd_head.argtypes = [i64, i64, vp, vp, vp, vp, dbl, i32, dbl, u64, i64, i64,
                                    vp, vp, vp, vp, vp]
    lib.oracle_bwd_head.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    return lib


def _f64(x) -> np.ndarray:
    """Exact up-cast to a C-contiguous float64 array (accepts torch tensors)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox-4x32-10 block for one 4-word counter and 2-word key."""
    lib = _load()
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def drop_threshold(p: float) -> int:
    return int(_load().oracle_drop_threshold(float(p)))


def keep_scale(p: float) -> float:
    return float(_load().oracle_keep_scale(float(p)))


def dropout_mask(N: int, p: float, seed: int, b: int, h: int) -> np.ndarray:
    """Keep mask (uint8, 1 = kept) of the (b, h) plane, shape [N, N]."""
    lib = _load()
    m = np.zeros((N, N), dtype=np.uint8)
    _check(lib.oracle_dropout_mask(N, float(p), seed & (2**64 - 1), b, h, _ptr(m)),
           "dropout_mask")
    return m


def fwd(q, k, v, scale: float, causal: bool = False, dropout_p: float = 0.0,
        seed: int = 0, heads=None):
    """O [B,H,N,d] and LSE [B,H,N] in float64.

    ``heads``: optional list of (b, h) pairs; only those heads are evaluated
    (the others are left as NaN).  ``k`` and ``v`` may have a different
    sequence length Nk than ``q`` (see oracle_fwd_cross for the causal rule).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    if k.shape[2] != N:
        return _fwd_cross(lib, q, k, v, scale, causal, dropout_p, seed, heads)
    o = np.full((B, H, N, d), np.nan)
    lse = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        ob = np.zeros((N, d))
        lb = np.zeros(N)
        _check(lib.oracle_fwd_rows(N, d, _ptr(q[b, h]), _ptr(k[b, h]), _ptr(v[b, h]),
                                   float(scale), int(bool(causal)), float(dropout_p),
                                   seed & (2**64 - 1), b, h, None, N, _ptr(ob), _ptr(lb)),
               "fwd")
        o[b, h] = ob
        lse[b, h] = lb
    return o, lse


def _fwd_cross(lib, q, k, v, scale, causal, dropout_p, seed, heads):
    """fwd for Nq != Nk, one oracle_fwd_cross call per head."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = np.full((B, H, Nq, d), np.nan)
    lse = np.full((B, H, Nq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        ob = np.zeros((Nq, d))
        lb = np.zeros(Nq)
        qh, kh, vh = (np.ascontiguousarray(x[b, h]) for x in (q, k, v))
        _check(lib.oracle_fwd_cross(Nq, Nk, d, _ptr(qh), _ptr(kh), _ptr(vh), float(scale),
                                    int(bool(causal)), float(dropout_p), seed & (2**64 - 1),
                                    b, h, _ptr(ob), _ptr(lb)), "fwd_cross")
        o[b, h] = ob
        lse[b, h] = lb
    return o, lse


def fwd_rows(q, k, v, b: int, h: int, rows, scale: float, causal: bool = False,
             dropout_p: float = 0.0, seed: int = 0):
    """O and LSE of selected rows of head (b, h): shapes [len(rows), d], [len(rows)].

    ``q``, ``k``, ``v`` are the full [B,H,N,d] tensors (only head (b, h) is read).
    """
    lib = _load()
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    N, d = qh.shape
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.zeros((len(r), d))
    lse = np.zeros(len(r))
    _check(lib.oracle_fwd_rows(N, d, _ptr(qh), _ptr(kh), _ptr(vh), float(scale),
                               int(bool(causal)), float(dropout_p), seed & (2**64 - 1),
                               b, h, _ptr(r), len(r), _ptr(o), _ptr(lse)), "fwd_rows")
    return o, lse


def probs(q, k, scale: float, causal: bool = False, dropout_p: float = 0.0,
          seed: int = 0, b: int = 0, h: int = 0):
    """(P, Pd) of one head given q, k of shape [N, d]: each [N, N] float64."""
    lib = _load()
    qh, kh = _f64(q), _f64(k)
    N, d = qh.shape
    P = np.zeros((N, N))
    Pd = np.zeros((N, N))
    _check(lib.oracle_probs(N, d, _ptr(qh), _ptr(kh), float(scale), int(bool(causal)),
                            float(dropout_p), seed & (2**64 - 1), b, h, _ptr(P), _ptr(Pd)),
           "probs")
    return P, Pd


def bwd(q, k, v, dout, scale: float, causal: bool = False, dropout_p: float = 0.0,
        seed: int = 0, heads=None):
    """(dq, dk, dv, o, lse) in float64 for [B,H,N,d] inputs.

    ``heads``: optional list of (b, h) pairs to evaluate (others stay NaN).
    """
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    if k.shape[2] != N:
        return _bwd_cross(lib, q, k, v, dout, scale, causal, dropout_p, seed, heads)
    outs = [np.full((B, H, N, d), np.nan) for _ in range(4)]
    lse = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        dq, dk, dv, o = (np.zeros((N, d)) for _ in range(4))
        lb = np.zeros(N)
        _check(lib.oracle_bwd_head(N, d, _ptr(q[b, h]), _ptr(k[b, h]), _ptr(v[b, h]),
                                   _ptr(dout[b, h]), float(scale), int(bool(causal)),
                                   float(dropout_p), seed & (2**64 - 1), b, h,
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(o), _ptr(lb)), "bwd")
        for dst, src in zip(outs, (dq, dk, dv, o)):
            dst[b, h] = src
        lse[b, h] = lb
    dq, dk, dv, o = outs
    return dq, dk, dv, o, lse


def bwd_one_head(q, k, v, dout, b: int, h: int, scale: float, causal: bool = False,
                 dropout_p: float = 0.0, seed: int = 0):
    """(dq, dk, dv, o, lse) in float64 of one head given as [N, d] arrays,
    with the dropout counters of head (b, h)."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    N, d = q.shape
    dq, dk, dv, o = (np.zeros((N, d)) for _ in range(4))
    lse = np.zeros(N)
    _check(lib.oracle_bwd_head(N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), float(scale),
                               int(bool(causal)), float(dropout_p), seed & (2**64 - 1), b, h,
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(o), _ptr(lse)), "bwd")
    return dq, dk, dv, o, lse


def _bwd_cross(lib, q, k, v, dout, scale, causal, dropout_p, seed, heads):
    """bwd for Nq != Nk (k, v [B,H,Nk,d]): dq, o [B,H,Nq,d]; dk, dv [B,H,Nk,d]."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dq_all, o_all = np.full((B, H, Nq, d), np.nan), np.full((B, H, Nq, d), np.nan)
    dk_all, dv_all = np.full((B, H, Nk, d), np.nan), np.full((B, H, Nk, d), np.nan)
    lse = np.full((B, H, Nq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        dq, o = np.zeros((Nq, d)), np.zeros((Nq, d))
        dk, dv = np.zeros((Nk, d)), np.zeros((Nk, d))
        lb = np.zeros(Nq)
        qh, kh, vh, dh = (np.ascontiguousarray(x[b, h]) for x in (q, k, v, dout))
        _check(lib.oracle_bwd_cross(Nq, Nk, d, _ptr(qh), _ptr(kh), _ptr(vh), _ptr(dh),
                                    float(scale), int(bool(causal)), float(dropout_p),
                                    seed & (2**64 - 1), b, h, _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(o), _ptr(lb)), "bwd_cross")
        dq_all[b, h], dk_all[b, h], dv_all[b, h], o_all[b, h] = dq, dk, dv, o
        lse[b, h] = lb
    return dq_all, dk_all, dv_all, o_all, lse
