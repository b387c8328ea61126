"""fp64 CPU oracle for the attention forward pass and its gradients.

TEST INFRASTRUCTURE. This package is the independent reference that the GPU
library is checked against. It shares no code with the GPU path and only the
test suite, the smoke check and the benchmark's CPU-baseline leg use it. It
never runs as part of the product.

Each function takes CPU tensors (torch or numpy) in any floating dtype,
up-converts them exactly to float64 and calls the C++ oracle in
``oracle.cpp``, which computes the textbook attention definition per output
row (scores, max-subtracted softmax, weighted sum of values; empty key set ->
O = 0, LSE = -inf). Results are float64 and unrounded.

``rows`` selects a subset of output rows (flattened indices); only those rows
are computed, which is how full-size workloads are checked on samples.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_attn_dense.argtypes = [P, P, I64, P, P, I64, I64, I64, I64, I64, I64, I64,
                                          P, P, P, P, ctypes.c_int, ctypes.c_double, P, P,
                                          ctypes.c_int]
        lib.oracle_attn_blocksparse.argtypes = [P, P, I64, P, P, I64, I64, I64, I64, I64, I64,
                                                I64, P, P, I64, I64, I64, P, ctypes.c_double,
                                                P, P, ctypes.c_int]
        lib.oracle_attn_topk.argtypes = [P, P, I64, P, P, I64, I64, I64, I64, I64, P, I64,
                                         ctypes.c_double, P, P, ctypes.c_int]
        lib.oracle_attn_dense_bwd.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, I64,
                                              P, P, P, P, ctypes.c_int, ctypes.c_double, P, P, P,
                                              ctypes.c_int]
        lib.oracle_attn_dense_bwd_bound.argtypes = lib.oracle_attn_dense_bwd.argtypes
        for f in (lib.oracle_attn_dense, lib.oracle_attn_blocksparse, lib.oracle_attn_topk,
                  lib.oracle_attn_dense_bwd, lib.oracle_attn_dense_bwd_bound):
            f.restype = ctypes.c_int
        lib.oracle_hardware_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


_ERRORS = {-1: "invalid argument", -2: "index out of range", -3: "duplicate index in a row"}


class OracleError(ValueError):
    pass


def _f64(x):
    """Exact up-conversion of a torch/numpy tensor to a C-contiguous float64 array."""
    if hasattr(x, "detach"):
        import torch
        return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x).astype(dtype, copy=False))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status):
    if status != 0:
        raise OracleError(_ERRORS.get(status, "oracle error %d" % status))


def hardware_threads() -> int:
    return _load().oracle_hardware_threads()


def _gather_rows(q, rows, width):
    """q viewed as [-1, width]; returns (q_rows float64, row_ids int64)."""
    flat = q.reshape(-1, width)
    if rows is None:
        ids = np.arange(flat.shape[0], dtype=np.int64)
        return _f64(flat), ids
    ids = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if hasattr(flat, "detach"):
        import torch
        sel = flat[torch.from_numpy(ids)]
    else:
        sel = np.asarray(flat)[ids]
    return _f64(sel), ids


def _mask_strides(mask, B, Hq, Sq, Skv):
    """uint8 mask of shape [Sq, Skv] or [B|1, Hq|1, Sq, Skv] -> (array, strides)."""
    m = _np(mask, np.uint8)
    if m.ndim == 2:
        if m.shape != (Sq, Skv):
            raise OracleError("mask shape %s" % (m.shape,))
        return m, np.array([0, 0, Skv, 1], dtype=np.int64)
    if m.ndim != 4 or m.shape[2:] != (Sq, Skv) or m.shape[0] not in (1, B) or m.shape[1] not in (1, Hq):
        raise OracleError("mask shape %s" % (m.shape,))
    st = [m.shape[1] * Sq * Skv, Sq * Skv, Skv, 1]
    if m.shape[0] == 1:
        st[0] = 0
    if m.shape[1] == 1:
        st[1] = 0
    return m, np.array(st, dtype=np.int64)


def attn_dense(q, k, v, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None,
               rows=None, nthreads=0):
    """Dense attention. q [B,Hq,Sq,D], k [B,Hkv,Skv,D], v [B,Hkv,Skv,Dv].

    Returns (o, lse): o [B,Hq,Sq,Dv] and lse [B,Hq,Sq] in float64, or
    [nrows, Dv] / [nrows] when ``rows`` (flattened (b,hq,i) ids) is given.
    ``scale`` is used as given (pass the float32 value the GPU receives).
    """
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, Dv = v.shape
    qr, ids = _gather_rows(q, rows, D)
    kk, vv = _f64(k), _f64(v)
    m, ms = (None, None) if mask is None else _mask_strides(mask, B, Hq, Sq, Skv)
    sq = _np(seqlens_q, np.int32)
    sk = _np(seqlens_k, np.int32)
    n = ids.shape[0]
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    _check(_load().oracle_attn_dense(_ptr(qr), _ptr(ids), n, _ptr(kk), _ptr(vv), B, Hq, Hkv, Sq,
                                     Skv, D, Dv, _ptr(m), _ptr(ms), _ptr(sq), _ptr(sk),
                                     int(bool(causal)), float(scale), _ptr(o), _ptr(lse),
                                     int(nthreads)))
    if rows is None:
        return o.reshape(B, Hq, Sq, Dv), lse.reshape(B, Hq, Sq)
    return o, lse


def attn_blocksparse(q, k, v, block_idx, *, scale, block_q=128, block_k=128, seqlens=None,
                     rows=None, nthreads=0):
    """Block-sparse attention. block_idx int32 [nQB, maxSel] (shared by every
    batch and KV head) or [B|1, Hkv|1, nQB, maxSel]; negative = unused slot."""
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, Dv = v.shape
    bi = _np(block_idx, np.int32)
    if bi.ndim == 2:
        bi = bi.reshape(1, 1, *bi.shape)
    if bi.ndim != 4 or bi.shape[0] not in (1, B) or bi.shape[1] not in (1, Hkv):
        raise OracleError("block_idx shape %s" % (bi.shape,))
    nqb_needed = (Sq + block_q - 1) // block_q
    if bi.shape[2] < nqb_needed:
        raise OracleError("block_idx has %d query blocks, need %d" % (bi.shape[2], nqb_needed))
    max_sel = bi.shape[3]
    bs = np.array([bi.shape[1] * bi.shape[2] * max_sel, bi.shape[2] * max_sel, max_sel, 1],
                  dtype=np.int64)
    if bi.shape[0] == 1:
        bs[0] = 0
    if bi.shape[1] == 1:
        bs[1] = 0
    qr, ids = _gather_rows(q, rows, D)
    kk, vv = _f64(k), _f64(v)
    sl = _np(seqlens, np.int32)
    n = ids.shape[0]
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    _check(_load().oracle_attn_blocksparse(_ptr(qr), _ptr(ids), n, _ptr(kk), _ptr(vv), B, Hq,
                                           Hkv, Sq, Skv, D, Dv, _ptr(bi), _ptr(bs), max_sel,
                                           block_q, block_k, _ptr(sl), float(scale), _ptr(o),
                                           _ptr(lse), int(nthreads)))
    if rows is None:
        return o.reshape(B, Hq, Sq, Dv), lse.reshape(B, Hq, Sq)
    return o, lse


def attn_topk(q, k, v, idx, *, scale, rows=None, nthreads=0):
    """Top-k gathered attention, one shared KV head.

    q [T,Hq,Dqk], k [S,Dqk], v [S,Dv], idx int32 [T,W] (negative = unused).
    Returns o [T,Hq,Dv], lse [T,Hq] (or [nrows,Dv], [nrows] with ``rows`` =
    flattened t*Hq+h ids)."""
    T, Hq, Dqk = q.shape
    S, Dv = v.shape
    if k.shape[0] != S or k.shape[1] != Dqk:
        raise OracleError("k shape %s" % (tuple(k.shape),))
    ii = _np(idx, np.int32)
    if ii.ndim != 2 or ii.shape[0] != T:
        raise OracleError("idx shape %s" % (ii.shape,))
    W = ii.shape[1]
    qr, ids = _gather_rows(q, rows, Dqk)
    kk, vv = _f64(k), _f64(v)
    n = ids.shape[0]
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    _check(_load().oracle_attn_topk(_ptr(qr), _ptr(ids), n, _ptr(kk), _ptr(vv), T, Hq, S, Dqk,
                                    Dv, _ptr(ii), W, float(scale), _ptr(o), _ptr(lse),
                                    int(nthreads)))
    if rows is None:
        return o.reshape(T, Hq, Dv), lse.reshape(T, Hq)
    return o, lse


def _bwd_call(fn, q, k, v, dout, scale, causal, mask, seqlens_q, seqlens_k, nthreads):
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, Dv = v.shape
    qa, ka, va, da = _f64(q), _f64(k), _f64(v), _f64(dout)
    m, ms = (None, None) if mask is None else _mask_strides(mask, B, Hq, Sq, Skv)
    sq, sk = _np(seqlens_q, np.int32), _np(seqlens_k, np.int32)
    gq = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    gk = np.zeros((B, Hkv, Skv, D), dtype=np.float64)
    gv = np.zeros((B, Hkv, Skv, Dv), dtype=np.float64)
    _check(fn(_ptr(qa), _ptr(ka), _ptr(va), _ptr(da), B, Hq, Hkv, Sq, Skv, D, Dv, _ptr(m), _ptr(ms), _ptr(sq),
              _ptr(sk), int(bool(causal)), float(scale), _ptr(gq), _ptr(gk), _ptr(gv), int(nthreads)))
    return gq, gk, gv


def attn_dense_bwd_bound(q, k, v, dout, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None,
                         nthreads=0):
    """First-order error scales (gq, gk, gv) of the gradients of dense
    attention, shaped like (dq, dk, dv): every signed sum of the gradient
    replaced by the sum of the magnitudes of its terms, plus the effect of an
    error of at most 2 E_i in the row term Delta_i (oracle.cpp states the
    formulas). A pipeline whose rounded quantities each carry a relative
    error <= u is within u times these of the exact gradients (first order)."""
    return _bwd_call(_load().oracle_attn_dense_bwd_bound, q, k, v, dout, scale, causal, mask, seqlens_q,
                     seqlens_k, nthreads)


def attn_dense_bwd(q, k, v, dout, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None,
                   nthreads=0):
    """Gradients (dq, dk, dv) of dense attention with respect to q, k, v given
    the output gradient dout [B,Hq,Sq,Dv]; same masking arguments as
    attn_dense. float64 numpy arrays shaped like q, k, v (dk, dv summed over
    the query heads of each KV head)."""
    return _bwd_call(_load().oracle_attn_dense_bwd, q, k, v, dout, scale, causal, mask, seqlens_q, seqlens_k,
                     nthreads)
