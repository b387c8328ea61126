"""Python binding of libfa.so, the gfx950 FlashAttention forward library.

Argument marshalling only: every step of the attention forward runs in the
HIP kernels behind the C ABI declared in include/fa.h. Tensors must be torch
tensors resident on the GPU; outputs are allocated with torch when not given.
Work is enqueued on torch's current stream. There is no CPU path: without the
built library or on a CPU tensor these functions raise.

Functions (same names as the C entry points):
  fa_fwd(q, k, v, scale=..., causal=False, mask=None, seqlens_q=None, seqlens_k=None,
         rescale_threshold=8.0)
  fa_fwd_blocksparse(q, k, v, block_idx, scale=..., block_q=128, block_k=128, seqlens=None,
                     rescale_threshold=8.0)
  fa_fwd_topk_gather(q, k, v, idx, scale=...)
each returning (o, lse).
"""
import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")
HEADER = os.path.join(HERE, "..", "include", "fa.h")

FA_F32, FA_F16, FA_BF16, FA_U8, FA_I32 = 0, 1, 2, 3, 4
_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16,
       torch.uint8: FA_U8, torch.bool: FA_U8, torch.int32: FA_I32}


class FaError(RuntimeError):
    def __init__(self, status, name, detail):
        super().__init__("%s: %s" % (name, detail))
        self.status = status
        self.name = name


class FaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


_lib = None


def declared_functions():
    """Names of the functions include/fa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status|const char\s*\*|int)\s+(fa_\w+)\s*\(", text, re.M)))


def load():
    """Loads libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FaError(-1, "FA_ERR_NOT_BUILT",
                          "%s is missing; build it with flashattention_online_softmax_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(FaTensor)
        lib.fa_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_float, ctypes.c_float, P, P,
                               ctypes.c_void_p]
        lib.fa_fwd_blocksparse.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_float,
                                           ctypes.c_float, P, P, ctypes.c_void_p]
        lib.fa_fwd_topk_gather.argtypes = [P, P, P, P, ctypes.c_float, P, P, ctypes.c_void_p]
        lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P, P, P, P, ctypes.c_void_p]
        for f in (lib.fa_fwd, lib.fa_fwd_blocksparse, lib.fa_fwd_topk_gather, lib.fa_bwd):
            f.restype = ctypes.c_int
        lib.fa_status_str.argtypes = [ctypes.c_int]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_last_error.argtypes = []
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def describe(t):
    """fa_tensor description of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % t.dtype)
    d = FaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = _DT[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _check(status):
    if status != 0:
        lib = load()
        raise FaError(status, lib.fa_status_str(status).decode(), lib.fa_last_error().decode())


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fa kernels take GPU tensors only (got a %s tensor)" % t.device)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# Rescale threshold (log2 units) of the dense and block-sparse entry points when
# none is given: the lazy default of the flash-attention forward described on the
# sparse-MLA page (threshold-branch section). 0 selects the exact running max.
DEFAULT_RESCALE_THRESHOLD = 8.0


def fa_fwd(q, k, v, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None,
           rescale_threshold=DEFAULT_RESCALE_THRESHOLD, out=None, lse=None, stream=None):
    """Dense/causal/masked/GQA attention forward. q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D];
    mask uint8/bool [Sq,Skv] or [B|1,Hq|1,Sq,Skv] (nonzero = excluded);
    rescale_threshold in [0, 10] (0 = exact running max)."""
    lib = load()
    _need_gpu(q, k, v, mask, seqlens_q, seqlens_k)
    B, Hq, Sq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, Sq, v.shape[3]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if mask is not None and mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _check(lib.fa_fwd(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(mask)),
                      _ref(describe(seqlens_q)), _ref(describe(seqlens_k)), int(bool(causal)),
                      float(scale), float(rescale_threshold), _ref(describe(out)), _ref(describe(lse)),
                      _stream(stream)))
    return out, lse


def fa_bwd(q, k, v, o, lse, dout, *, scale, causal=False, mask=None, dq=None, dk=None, dv=None, delta=None,
           stream=None):
    """Gradients (dq, dk, dv) of the dense/causal/masked/GQA forward given
    its output o, its lse and the output gradient dout (f16/bf16, D = 128);
    mask as fa_fwd's (uint8, non-zero = excluded).
    delta (fp32 [B,Hq,Sq]) is the kernels' workspace; it is allocated here
    when not given."""
    lib = load()
    _need_gpu(q, k, v, o, lse, dout, mask)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if delta is None:
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib.fa_bwd(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(mask)), _ref(describe(o)),
                      _ref(describe(lse)), _ref(describe(dout)), int(bool(causal)), float(scale),
                      _ref(describe(delta)), _ref(describe(dq)), _ref(describe(dk)), _ref(describe(dv)),
                      _stream(stream)))
    return dq, dk, dv


def fa_fwd_blocksparse(q, k, v, block_idx, *, scale, block_q=128, block_k=128, seqlens=None,
                       rescale_threshold=DEFAULT_RESCALE_THRESHOLD, out=None, lse=None, stream=None):
    """Block-sparse attention forward; block_idx int32 [nQB, maxSel] or
    [B|1, Hkv|1, nQB, maxSel], negative = unused slot."""
    lib = load()
    _need_gpu(q, k, v, block_idx, seqlens)
    B, Hq, Sq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, Sq, v.shape[3]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_blocksparse(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)),
                                  _ref(describe(block_idx)), int(block_q), int(block_k),
                                  _ref(describe(seqlens)), float(scale), float(rescale_threshold),
                                  _ref(describe(out)), _ref(describe(lse)), _stream(stream)))
    return out, lse


def fa_fwd_topk_gather(q, k, v, idx, *, scale, out=None, lse=None, stream=None):
    """Top-k gathered MLA attention forward. q [T,Hq,Dqk], k [S,Dqk], v [S,Dv]
    (v may be k[:, :Dv]), idx int32 [T,W] (negative = unused)."""
    lib = load()
    _need_gpu(q, k, v, idx)
    T, Hq, _ = q.shape
    if out is None:
        out = torch.empty((T, Hq, v.shape[1]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_topk_gather(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)),
                                  _ref(describe(idx)), float(scale), _ref(describe(out)),
                                  _ref(describe(lse)), _stream(stream)))
    return out, lse


def version():
    return load().fa_version()
