"""Python binding of libfa.so, the gfx950 FlashAttention forward library.

Argument marshalling only: every step of the attention forward runs in the
HIP kernels behind the C ABI declared in include/fa.h. Tensors must be torch
tensors resident on the GPU; outputs are allocated with torch when not given.
Work is enqueued on torch's current stream. There is no CPU path: without the
built library or on a CPU tensor these functions raise.

Functions (same names as the C entry points):
  fa_fwd(q, k, v, scale=..., causal=False, mask=None, seqlens_q=None, seqlens_k=None,
         rescale_threshold=0.0)
  fa_fwd_blocksparse(q, k, v, block_idx, scale=..., block_q=128, block_k=128, seqlens=None,
                     rescale_threshold=0.0)
  fa_fwd_topk_gather(q, k, v, idx, scale=...)
each returning (o, lse); also fa_fwd_varlen, fa_fwd_splitkv(_noalloc) and the
backward fa_bwd / fa_bwd_varlen, returning (dq, dk, dv).
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
    return sorted(set(re.findall(r"^\s*(?:fa_status|const char\s*\*|int|int64_t)\s+(fa_\w+)\s*\(", text, re.M)))


def load():
    """Loads libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FaError(-1, "FA_ERR_NOT_BUILT",
                          "%s is missing; build it with flashattention_online_softmax_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(FaTensor)
        lib.fa_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_float, ctypes.c_float, P, P, P,
                               ctypes.c_void_p]
        lib.fa_fwd_blocksparse.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, P, ctypes.c_float,
                                           ctypes.c_float, P, P, ctypes.c_void_p]
        lib.fa_fwd_topk_gather.argtypes = [P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_void_p]
        lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P, P, P, P, P,
                               ctypes.c_void_p]
        lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                      P, P, ctypes.c_void_p]
        lib.fa_bwd_varlen.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, ctypes.c_int,
                                      ctypes.c_float, P, P, P, P, P, ctypes.c_void_p]
        lib.fa_bwd_ds_workspace_elems.argtypes = [ctypes.c_int64] * 4
        lib.fa_bwd_ds_workspace_elems.restype = ctypes.c_int64
        lib.fa_fwd_splitkv.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                       P, P, P, ctypes.c_void_p]
        lib.fa_fwd_splitkv_noalloc.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                               ctypes.c_int, P, P, ctypes.c_void_p]
        lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
        lib.fa_fwd_splitkv_splits.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
        lib.fa_fwd_splitkv_splits.restype = ctypes.c_int
        lib.fa_fwd_splitkv_workspace_elems.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int]
        lib.fa_fwd_splitkv_workspace_elems.restype = ctypes.c_int64
        for f in (lib.fa_fwd, lib.fa_fwd_blocksparse, lib.fa_fwd_topk_gather, lib.fa_bwd, lib.fa_fwd_varlen,
                  lib.fa_fwd_splitkv, lib.fa_bwd_varlen):
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
# none is given: 0, the exact running max (a row's reference max moves on every
# growth, so its largest weight is exactly 1 before P.V). The lazy rescale of the
# flash-attention sparse-MLA page (threshold-branch section) is the opt-in
# rescale_threshold=8.
DEFAULT_RESCALE_THRESHOLD = 0.0


def _o_lo(want, o_lo, out):
    """The fp32 rounding-residual output: the caller's tensor, a new one when
    asked for (want=True), or None."""
    if o_lo is not None:
        return o_lo
    if want:
        return torch.empty(out.shape, dtype=torch.float32, device=out.device)
    return None


def fa_fwd(q, k, v, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None,
           rescale_threshold=DEFAULT_RESCALE_THRESHOLD, out=None, lse=None, return_o_lo=False, o_lo=None,
           stream=None):
    """Dense/causal/masked/GQA attention forward. q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D];
    mask uint8/bool [Sq,Skv] or [B|1,Hq|1,Sq,Skv] (nonzero = excluded);
    rescale_threshold in [0, 10] (0 = exact running max). Returns (o, lse),
    or (o, lse, o_lo) with return_o_lo / o_lo given: o_lo = fp32(O) - o,
    the output's rounding residual."""
    lib = load()
    _need_gpu(q, k, v, mask, seqlens_q, seqlens_k, o_lo)
    B, Hq, Sq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, Sq, v.shape[3]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if mask is not None and mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    lo = _o_lo(return_o_lo, o_lo, out)
    _check(lib.fa_fwd(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(mask)),
                      _ref(describe(seqlens_q)), _ref(describe(seqlens_k)), int(bool(causal)),
                      float(scale), float(rescale_threshold), _ref(describe(out)), _ref(describe(lo)),
                      _ref(describe(lse)), _stream(stream)))
    return (out, lse) if lo is None else (out, lse, lo)


# The stored-dS backward path (dQ from the dS the dK/dV kernel stores)
# against the recomputing one, measured on MI355X (causal bf16, D = 128):
# faster while the dS the sweep touches fits the 256 MB last-level cache
# (B = 2, H = 16: S = 1024 -18%, S = 2048 -11%) and while batch x heads is too
# small to fill the GPU several times, where the longest workgroups set the
# time (B = 1: H = 8 S = 4096 -23%, H = 4 S = 8192 -22%); on large, full
# problems (B = 2, H = 16, S = 4096 / 8192) the two are within the 2-4% the
# hosts differ by. "auto" takes it when the touched dS (half of the blocks
# under the causal mask) is at most DS_AUTO_TOUCHED_BYTES or the dK/dV grid
# (B Hkv ceil(Skv / 128) workgroups) is below DS_AUTO_FULL_GRID, and the
# workspace stays within DS_WORKSPACE_MAX_BYTES.
DS_AUTO_TOUCHED_BYTES = 160 << 20
DS_AUTO_FULL_GRID = 1024
DS_WORKSPACE_MAX_BYTES = 8 << 30


def _ds_work(q, B, Hq, Hkv, Sq, Skv, ws, causal):
    """The dS workspace argument of the backward: "auto" allocates one when
    the stored-dS path is expected to be the faster one (see above), True
    always, None or False never (the dQ kernel recomputes S and dP); a tensor
    is passed through."""
    if ws is None or ws is False:
        return None
    if ws is True or isinstance(ws, str):
        if ws is not True and ws != "auto":
            raise ValueError("ds_workspace must be 'auto', True, None or a tensor")
        n = load().fa_bwd_ds_workspace_elems(B, Hq, Sq, Skv)
        if n <= 0:
            return None
        if ws == "auto":
            touched = 2 * B * Hq * ((Sq + 255) // 256 * 256) * ((Skv + 31) // 32 * 32) // (2 if causal else 1)
            grid = B * Hkv * ((Skv + 127) // 128)
            if 2 * n > DS_WORKSPACE_MAX_BYTES or (touched > DS_AUTO_TOUCHED_BYTES and grid >= DS_AUTO_FULL_GRID):
                return None
        return torch.empty(n, dtype=q.dtype, device=q.device)
    return ws


def ds_workspace_elems(B, Hq, Sq, Skv):
    """Elements of the backward's dS workspace for these sizes."""
    return load().fa_bwd_ds_workspace_elems(B, Hq, Sq, Skv)


def fa_bwd(q, k, v, o, lse, dout, *, scale, causal=False, mask=None, seqlens_q=None, seqlens_k=None, o_lo=None,
           dq=None, dk=None, dv=None, delta=None, ds_workspace="auto", stream=None):
    """Gradients (dq, dk, dv) of the dense/causal/masked/GQA forward given
    its output o, its lse and the output gradient dout (f16/bf16, D = 64 or 128);
    mask and sequence lengths as fa_fwd's; o_lo (the forward's rounding
    residual) makes Delta = dO . (o + o_lo).
    delta (fp32 [B,Hq,Sq]) is the kernels' workspace; it is allocated here
    when not given. ds_workspace: "auto" (dQ from the stored dS where that
    path is the faster one, see DS_AUTO_TOUCHED_BYTES), True (always), None
    (dQ recomputes S and dP) or a tensor of fa_bwd_ds_workspace_elems
    elements in q's dtype."""
    lib = load()
    _need_gpu(q, k, v, o, lse, dout, mask, seqlens_q, seqlens_k, o_lo)
    ws = _ds_work(q, q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2], ds_workspace, causal)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if delta is None:
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if mask is not None and mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _check(lib.fa_bwd(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(mask)),
                      _ref(describe(seqlens_q)), _ref(describe(seqlens_k)), _ref(describe(o)), _ref(describe(o_lo)),
                      _ref(describe(lse)), _ref(describe(dout)), int(bool(causal)), float(scale),
                      _ref(describe(delta)), _ref(describe(dq)), _ref(describe(dk)), _ref(describe(dv)),
                      _ref(describe(ws)), _stream(stream)))
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


def fa_fwd_topk_gather(q, k, v, idx, *, scale, out=None, lse=None, return_o_lo=False, o_lo=None, stream=None):
    """Top-k gathered MLA attention forward. q [T,Hq,Dqk], k [S,Dqk], v [S,Dv]
    (v may be k[:, :Dv]), idx int32 [T,W] (negative = unused). Returns
    (o, lse), or (o, lse, o_lo) as fa_fwd."""
    lib = load()
    _need_gpu(q, k, v, idx, o_lo)
    T, Hq, _ = q.shape
    if out is None:
        out = torch.empty((T, Hq, v.shape[1]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    lo = _o_lo(return_o_lo, o_lo, out)
    _check(lib.fa_fwd_topk_gather(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)),
                                  _ref(describe(idx)), float(scale), _ref(describe(out)), _ref(describe(lo)),
                                  _ref(describe(lse)), _stream(stream)))
    return (out, lse) if lo is None else (out, lse, lo)


def version():
    return load().fa_version()


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, *, scale, causal=False,
                  rescale_threshold=DEFAULT_RESCALE_THRESHOLD, out=None, lse=None, stream=None):
    """Packed variable-length (TND) forward: q [Tq,Hq,D], k/v [Tk,Hkv,D],
    cu_seqlens_q / cu_seqlens_k int32 [B+1] on the GPU; returns (o [Tq,Hq,Dv],
    lse [Tq,Hq])."""
    lib = load()
    _need_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if out is None:
        out = torch.zeros((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.full((q.shape[0], q.shape[1]), float("-inf"), dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_varlen(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(cu_seqlens_q)),
                             _ref(describe(cu_seqlens_k)), int(max_seqlen_q), int(bool(causal)), float(scale),
                             float(rescale_threshold), _ref(describe(out)), _ref(describe(lse)), _stream(stream)))
    return out, lse


def fa_bwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, o, lse, dout, *, scale,
                  causal=False, o_lo=None, dq=None, dk=None, dv=None, delta=None, ds_workspace="auto", stream=None):
    """Gradients (dq, dk, dv) of the packed variable-length (TND) forward:
    q [Tq,Hq,D], k/v [Tk,Hkv,D], cu_seqlens int32 [B+1] on the GPU, o / lse
    from fa_fwd_varlen, dout [Tq,Hq,Dv]. Rows and keys outside every sequence
    are not written (the outputs allocated here start as zeros).
    ds_workspace as fa_bwd's (sized for B sequences of the longest lengths)."""
    lib = load()
    _need_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, dout, o_lo)
    ws = _ds_work(q, cu_seqlens_q.shape[0] - 1, q.shape[1], k.shape[1], int(max_seqlen_q), int(max_seqlen_k),
                  ds_workspace, causal)
    if dq is None:
        dq = torch.zeros_like(q)
    if dk is None:
        dk = torch.zeros_like(k)
    if dv is None:
        dv = torch.zeros_like(v)
    if delta is None:
        delta = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _check(lib.fa_bwd_varlen(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(cu_seqlens_q)),
                             _ref(describe(cu_seqlens_k)), int(max_seqlen_q), int(max_seqlen_k), _ref(describe(o)),
                             _ref(describe(o_lo)), _ref(describe(lse)), _ref(describe(dout)), int(bool(causal)),
                             float(scale), _ref(describe(delta)), _ref(describe(dq)), _ref(describe(dk)),
                             _ref(describe(dv)), _ref(describe(ws)), _stream(stream)))
    return dq, dk, dv


def splitkv_splits(B, Hq, Sq, Skv, num_splits=0):
    """Number of key ranges fa_fwd_splitkv uses for these sizes."""
    return load().fa_fwd_splitkv_splits(B, Hq, Sq, Skv, num_splits)


def fa_fwd_splitkv(q, k, v, *, scale, causal=False, seqlens_q=None, seqlens_k=None, num_splits=0,
                   rescale_threshold=DEFAULT_RESCALE_THRESHOLD, workspace=None, out=None, lse=None, stream=None):
    """Split-KV forward (fa_fwd's semantics, for few rows over many keys); the
    fp32 workspace is allocated here when not given."""
    lib = load()
    _need_gpu(q, k, v, seqlens_q, seqlens_k, workspace)
    B, Hq, Sq, _ = q.shape
    Skv, Dv = k.shape[2], v.shape[3]
    if out is None:
        out = torch.empty((B, Hq, Sq, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = lib.fa_fwd_splitkv_workspace_elems(B, Hq, Sq, Skv, Dv, int(num_splits))
        if n > 0:
            workspace = torch.empty(n, dtype=torch.float32, device=q.device)
    _check(lib.fa_fwd_splitkv(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)), _ref(describe(seqlens_q)),
                              _ref(describe(seqlens_k)), int(bool(causal)), float(scale), float(rescale_threshold),
                              int(num_splits), _ref(describe(workspace)), _ref(describe(out)), _ref(describe(lse)),
                              _stream(stream)))
    return out, lse


def fa_fwd_splitkv_noalloc(q, k, v, *, scale, causal=False, seqlens_q=None, seqlens_k=None, num_splits=0,
                           rescale_threshold=DEFAULT_RESCALE_THRESHOLD, out, lse, stream=None):
    """fa_fwd_splitkv whose partial results live in the library's static
    device scratch (no allocation in the call; out and lse are required)."""
    lib = load()
    _need_gpu(q, k, v, seqlens_q, seqlens_k, out, lse)
    _check(lib.fa_fwd_splitkv_noalloc(_ref(describe(q)), _ref(describe(k)), _ref(describe(v)),
                                      _ref(describe(seqlens_q)), _ref(describe(seqlens_k)), int(bool(causal)),
                                      float(scale), float(rescale_threshold), int(num_splits), _ref(describe(out)),
                                      _ref(describe(lse)), _stream(stream)))
    return out, lse
