"""CPU checks of the C ABI: the library loads, exports every function that
include/fa.h declares, and rejects invalid arguments on the host before any
launch (no GPU is touched: every call here fails validation or is empty)."""
import ctypes
import math
import os

import pytest
import numpy as np
import torch

import flashattention_online_softmax_amd as fa

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from flashattention_online_softmax_amd import build
        build.build()
    return fa.load()


def T(shape, dtype=fa.FA_BF16, stride=None, data=FAKE):
    t = fa.FaTensor()
    t.data = data
    t.dtype = dtype
    t.ndim = len(shape)
    if stride is None:
        stride, s = [], 1
        for n in reversed(shape):
            stride.insert(0, s)
            s *= n
    for i, (n, st) in enumerate(zip(shape, stride)):
        t.shape[i] = n
        t.stride[i] = st
    return t


def R(t):
    return None if t is None else ctypes.byref(t)


def name(lib, s):
    return lib.fa_status_str(s).decode()


def call_fwd(lib, q, k, v, o, lse, mask=None, sq=None, sk=None, causal=0, scale=0.1, thr=0.0, o_lo=None):
    return name(lib, lib.fa_fwd(R(q), R(k), R(v), R(mask), R(sq), R(sk), causal, scale, thr, R(o), R(o_lo),
                                R(lse), None))


def good(B=2, Hq=4, Hkv=2, S=64, D=128, dt=fa.FA_BF16):
    return (T([B, Hq, S, D], dt), T([B, Hkv, S, D], dt), T([B, Hkv, S, D], dt),
            T([B, Hq, S, D], dt), T([B, Hq, S], fa.FA_F32))


def test_exports_every_declared_function(lib):
    names = fa.declared_functions()
    assert {"fa_fwd", "fa_fwd_blocksparse", "fa_fwd_topk_gather", "fa_bwd", "fa_fwd_varlen", "fa_bwd_varlen",
            "fa_bwd_ds_workspace_elems", "fa_fwd_splitkv", "fa_fwd_splitkv_splits",
            "fa_fwd_splitkv_workspace_elems", "fa_status_str", "fa_last_error", "fa_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fa_version() == 400  # 0.4.0: the backward entry points take a dS workspace


def test_status_names(lib):
    assert [name(lib, i) for i in range(8)] == [
        "FA_OK", "FA_ERR_NULL", "FA_ERR_DTYPE", "FA_ERR_SHAPE", "FA_ERR_STRIDE",
        "FA_ERR_UNSUPPORTED", "FA_ERR_VALUE", "FA_ERR_HIP"]


def test_fa_fwd_validation(lib):
    q, k, v, o, lse = good()
    assert call_fwd(lib, None, k, v, o, lse) == "FA_ERR_NULL"
    assert call_fwd(lib, q, k, v, o, lse, causal=2) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, k, v, o, lse, scale=float("nan")) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, k, v, o, lse, scale=-1.0) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, k, v, o, lse, scale=0.0) == "FA_ERR_VALUE"
    # rescale threshold: [0, 10] log2 units
    assert call_fwd(lib, q, k, v, o, lse, thr=-0.5) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, k, v, o, lse, thr=10.5) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, k, v, o, lse, thr=float("nan")) == "FA_ERR_VALUE"
    assert call_fwd(lib, q, T([2, 2, 64, 128], fa.FA_F16), v, o, lse) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, k, v, o, T([2, 4, 64], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, T([2, 3, 64, 128]), T([2, 3, 64, 128]), o, lse) == "FA_ERR_SHAPE"
    assert b"multiple of Hkv" in lib.fa_last_error()
    assert call_fwd(lib, *good(D=96)) == "FA_ERR_UNSUPPORTED"
    assert call_fwd(lib, *good(dt=fa.FA_I32)) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, k, v, T([2, 4, 64, 64]), lse) == "FA_ERR_SHAPE"
    assert call_fwd(lib, q, k, v, o, T([2, 4, 64], fa.FA_F32, stride=[512, 1, 4])) == "FA_ERR_STRIDE"
    # last dim not contiguous / misaligned pointer / misaligned row stride
    assert call_fwd(lib, T([2, 4, 64, 128], stride=[65536, 16384, 256, 2]), k, v, o, lse) == "FA_ERR_STRIDE"
    assert call_fwd(lib, T([2, 4, 64, 128], data=FAKE + 2), k, v, o, lse) == "FA_ERR_STRIDE"
    assert call_fwd(lib, T([2, 4, 64, 128], stride=[4 * 64 * 130, 64 * 130, 130, 1]), k, v, o, lse) == "FA_ERR_STRIDE"
    # mask / seqlens
    assert call_fwd(lib, q, k, v, o, lse, mask=T([64, 64], fa.FA_F16)) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, k, v, o, lse, mask=T([64, 63], fa.FA_U8)) == "FA_ERR_SHAPE"
    assert call_fwd(lib, q, k, v, o, lse, mask=T([3, 1, 64, 64], fa.FA_U8)) == "FA_ERR_SHAPE"
    assert call_fwd(lib, q, k, v, o, lse, sq=T([2], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, k, v, o, lse, sk=T([3], fa.FA_I32)) == "FA_ERR_SHAPE"
    # o_lo: fp32, shaped like o, 16-bit outputs only
    assert call_fwd(lib, q, k, v, o, lse, o_lo=T([2, 4, 64, 128], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert call_fwd(lib, q, k, v, o, lse, o_lo=T([2, 4, 64, 64], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert call_fwd(lib, q, k, v, o, lse, o_lo=T([2, 4, 64, 128], fa.FA_F32, data=FAKE + 4)) == "FA_ERR_STRIDE"
    q32, k32, v32, o32, l32 = good(dt=fa.FA_F32)
    assert call_fwd(lib, q32, k32, v32, o32, l32, o_lo=T([2, 4, 64, 128], fa.FA_F32)) == "FA_ERR_UNSUPPORTED"


def test_empty_problems_launch_nothing(lib):
    # no output rows: FA_OK without touching the device (no GPU here)
    assert call_fwd(lib, *good(B=0)) == "FA_OK"
    q, k, v, o, lse = good(S=0)
    assert call_fwd(lib, q, k, v, o, lse) == "FA_OK"
    assert lib.fa_last_error() == b""


def test_blocksparse_validation(lib):
    q, k, v, o, lse = good(S=256)
    bi = T([2, 16], fa.FA_I32)

    def bs(bi=bi, bq=128, bk=128, seq=None, q=q, thr=8.0):
        return name(lib, lib.fa_fwd_blocksparse(R(q), R(k), R(v), R(bi), bq, bk, R(seq), 0.1, thr, R(o),
                                                R(lse), None))

    assert bs(bq=64) == "FA_ERR_UNSUPPORTED"
    assert bs(bi=None) == "FA_ERR_NULL"
    assert bs(bi=T([1, 16], fa.FA_I32)) == "FA_ERR_SHAPE"  # too few query blocks
    assert bs(bi=T([2, 300], fa.FA_I32)) == "FA_ERR_UNSUPPORTED"
    assert bs(bi=T([2, 16], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert bs(bi=T([3, 2, 2, 16], fa.FA_I32)) == "FA_ERR_SHAPE"
    assert bs(seq=T([2], fa.FA_U8)) == "FA_ERR_DTYPE"
    assert bs(thr=-1.0) == "FA_ERR_VALUE"
    q0, k0, v0, o0, l0 = good(B=0, S=256)
    assert name(lib, lib.fa_fwd_blocksparse(R(q0), R(k0), R(v0), R(bi), 128, 128, None, 0.1, 0.0, R(o0),
                                            R(l0), None)) == "FA_OK"


def test_topk_validation(lib):
    def tk(q=T([8, 128, 576]), k=T([16, 576]), v=None, idx=T([8, 32], fa.FA_I32),
           o=T([8, 128, 512]), lse=T([8, 128], fa.FA_F32), scale=0.04, o_lo=None):
        if v is None:
            v = T([16, 512], stride=[576, 1])
        return name(lib, lib.fa_fwd_topk_gather(R(q), R(k), R(v), R(idx), scale, R(o), R(o_lo), R(lse), None))

    assert tk(q=T([8, 128, 576], fa.FA_F32), k=T([16, 576], fa.FA_F32), v=T([16, 512], fa.FA_F32),
              o=T([8, 128, 512], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert tk(idx=T([8, 32], fa.FA_U8)) == "FA_ERR_DTYPE"
    assert tk(q=T([8, 128, 512]), k=T([16, 512])) == "FA_ERR_UNSUPPORTED"
    assert tk(o_lo=T([8, 128, 512], fa.FA_F16)) == "FA_ERR_DTYPE"
    assert tk(o_lo=T([8, 100, 512], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert tk(idx=T([8, 5000], fa.FA_I32)) == "FA_ERR_UNSUPPORTED"
    assert tk(idx=T([7, 32], fa.FA_I32)) == "FA_ERR_SHAPE"
    assert tk(v=T([15, 512])) == "FA_ERR_SHAPE"
    assert tk(scale=float("inf")) == "FA_ERR_VALUE"
    assert tk(q=T([0, 128, 576]), idx=T([0, 32], fa.FA_I32), o=T([0, 128, 512]),
              lse=T([0, 128], fa.FA_F32)) == "FA_OK"


def test_bwd_ds_workspace_policy(lib):
    # "auto" takes the stored-dS path while the dS it touches (half of the
    # blocks under the causal mask) fits the cache or the dK/dV grid is below
    # four rounds of the GPU; True always, None never. (CPU tensors: only the
    # sizing decision is exercised here.)
    q = torch.empty(0, dtype=torch.bfloat16)
    assert fa._ds_work(q, 2, 16, 16, 1024, 1024, "auto", True) is not None
    assert fa._ds_work(q, 2, 16, 16, 2048, 2048, "auto", True) is not None    # 134 MB touched
    assert fa._ds_work(q, 4, 16, 16, 2048, 2048, "auto", True) is None        # 268 MB, 1024 workgroups
    assert fa._ds_work(q, 2, 16, 16, 4096, 4096, "auto", True) is None        # 537 MB, 1024 workgroups
    assert fa._ds_work(q, 1, 4, 4, 8192, 8192, "auto", True) is not None      # 268 MB, 256 workgroups
    assert fa._ds_work(q, 2, 32, 8, 4096, 4096, "auto", True) is not None     # GQA: 512 workgroups
    assert fa._ds_work(q, 1, 2, 2, 100000, 100000, "auto", True) is None      # workspace above the cap
    w = fa._ds_work(q, 1, 2, 2, 100, 70, True, False)
    assert w.numel() == lib.fa_bwd_ds_workspace_elems(1, 2, 100, 70) and w.dtype == torch.bfloat16
    assert fa._ds_work(q, 1, 2, 2, 100, 70, None, False) is None
    with pytest.raises(ValueError):
        fa._ds_work(q, 1, 2, 2, 100, 70, "always", False)


def test_bwd_validation(lib):
    def bw(dt=fa.FA_BF16, D=128, dq_shape=None, delta_dt=fa.FA_F32, B=2, causal=1, mask=None, sq=None, sk=None,
           o_lo=None, ds=None):
        q, k, v, o, lse = good(B=B, D=D, dt=dt)
        dout = T([B, 4, 64, D], dt)
        dq = T(dq_shape or [B, 4, 64, D], dt)
        dk, dv = T([B, 2, 64, D], dt), T([B, 2, 64, D], dt)
        delta = T([B, 4, 64], delta_dt)
        return name(lib, lib.fa_bwd(R(q), R(k), R(v), R(mask), R(sq), R(sk), R(o), R(o_lo), R(lse), R(dout), causal,
                                    0.1, R(delta), R(dq), R(dk), R(dv), R(ds), None))

    assert bw(dt=fa.FA_F32) == "FA_ERR_UNSUPPORTED"
    assert bw(D=96) == "FA_ERR_UNSUPPORTED"
    assert bw(D=64, B=0) == "FA_OK"  # head dim 64 is accepted
    assert bw(dq_shape=[2, 4, 63, 128]) == "FA_ERR_SHAPE"
    assert bw(delta_dt=fa.FA_BF16) == "FA_ERR_DTYPE"
    assert bw(causal=2) == "FA_ERR_VALUE"
    assert bw(mask=T([64, 63], fa.FA_U8)) == "FA_ERR_SHAPE"
    assert bw(mask=T([3, 4, 64, 64], fa.FA_U8)) == "FA_ERR_SHAPE"
    assert bw(mask=T([64, 64], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert bw(sq=T([3], fa.FA_I32)) == "FA_ERR_SHAPE"
    assert bw(sk=T([2], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert bw(o_lo=T([2, 4, 64, 128], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert bw(o_lo=T([2, 4, 63, 128], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert bw(B=0) == "FA_OK"  # nothing to do: no launch
    # dS workspace: B * Hq * (Sq256 * Skv32 + 4 * Sq32) elements (dS blocks,
    # then two fp32 start values per row)
    n = lib.fa_bwd_ds_workspace_elems(2, 4, 64, 64)
    assert n == 2 * 4 * (256 * 64 + 4 * 64)
    assert lib.fa_bwd_ds_workspace_elems(1, 1, 33, 70) == 256 * 96 + 4 * 64
    assert lib.fa_bwd_ds_workspace_elems(-1, 1, 1, 1) == -1
    assert bw(ds=T([n - 1])) == "FA_ERR_SHAPE"
    assert b"ds_workspace holds" in lib.fa_last_error()
    assert bw(ds=T([n], fa.FA_F16)) == "FA_ERR_DTYPE"
    assert bw(ds=T([n], data=FAKE + 8)) == "FA_ERR_STRIDE"
    assert bw(ds=T([n]), B=0) == "FA_OK"


def test_varlen_validation(lib):
    def vl(q=T([100, 4, 128]), k=T([120, 2, 128]), v=T([120, 2, 128]), cq=T([4], fa.FA_I32), ck=T([4], fa.FA_I32),
           maxq=50, o=T([100, 4, 128]), lse=T([100, 4], fa.FA_F32), causal=1, thr=0.0):
        return name(lib, lib.fa_fwd_varlen(R(q), R(k), R(v), R(cq), R(ck), maxq, causal, 0.1, thr, R(o), R(lse), None))

    assert vl(q=T([100, 4, 128], fa.FA_F32), k=T([120, 2, 128], fa.FA_F32), v=T([120, 2, 128], fa.FA_F32),
              o=T([100, 4, 128], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert vl(cq=T([4], fa.FA_I32), ck=T([5], fa.FA_I32)) == "FA_ERR_SHAPE"
    assert vl(cq=T([0], fa.FA_I32), ck=T([0], fa.FA_I32)) == "FA_ERR_SHAPE"
    assert vl(cq=T([4], fa.FA_F32)) == "FA_ERR_DTYPE"
    assert vl(k=T([120, 3, 128]), v=T([120, 3, 128])) == "FA_ERR_SHAPE"
    assert vl(v=T([119, 2, 128])) == "FA_ERR_SHAPE"
    assert vl(lse=T([100, 3], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert vl(maxq=-1) == "FA_ERR_VALUE"
    assert vl(causal=3) == "FA_ERR_VALUE"
    assert vl(thr=11.0) == "FA_ERR_VALUE"
    assert vl(q=T([100, 4, 96]), k=T([120, 2, 96]), v=T([120, 2, 96]), o=T([100, 4, 96])) == "FA_ERR_UNSUPPORTED"
    assert vl(maxq=0) == "FA_OK"  # no rows: nothing launched
    assert vl(cq=T([1], fa.FA_I32), ck=T([1], fa.FA_I32)) == "FA_OK"  # B = 0


def test_bwd_varlen_validation(lib):
    def bv(Tq=100, Tk=120, Hq=4, Hkv=2, D=128, dt=fa.FA_BF16, nb=4, nbk=None, maxq=50, maxk=60, causal=1,
           scale=0.1, lse=None, delta=None, o_lo=None, dk=None, q_stride=None, ds=None):
        q = T([Tq, Hq, D], dt, stride=q_stride)
        kk = T([Tk, Hkv, D], dt)
        lse = T([Tq, Hq], fa.FA_F32) if lse is None else lse
        delta = T([Tq, Hq], fa.FA_F32) if delta is None else delta
        dk = T([Tk, Hkv, D], dt) if dk is None else dk
        return name(lib, lib.fa_bwd_varlen(R(q), R(kk), R(T([Tk, Hkv, D], dt)), R(T([nb], fa.FA_I32)),
                                           R(T([nb if nbk is None else nbk], fa.FA_I32)), maxq, maxk,
                                           R(T([Tq, Hq, D], dt)), R(o_lo), R(lse), R(T([Tq, Hq, D], dt)), causal,
                                           scale, R(delta), R(T([Tq, Hq, D], dt)), R(dk), R(T([Tk, Hkv, D], dt)),
                                           R(ds), None))

    assert bv(dt=fa.FA_F32) == "FA_ERR_DTYPE"
    assert bv(nbk=5) == "FA_ERR_SHAPE"
    assert bv(nb=0, nbk=0) == "FA_ERR_SHAPE"
    assert bv(Hkv=3) == "FA_ERR_SHAPE"
    assert bv(lse=T([100, 3], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert bv(delta=T([100, 4], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert bv(delta=T([100, 4], fa.FA_F32, stride=[8, 1])) == "FA_ERR_STRIDE"
    assert bv(dk=T([119, 2, 128])) == "FA_ERR_SHAPE"
    assert bv(o_lo=T([100, 4, 128], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert bv(o_lo=T([99, 4, 128], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert bv(maxq=-1) == "FA_ERR_VALUE"
    assert bv(maxk=-1) == "FA_ERR_VALUE"
    assert bv(causal=2) == "FA_ERR_VALUE"
    assert bv(scale=float("inf")) == "FA_ERR_VALUE"
    assert bv(D=96) == "FA_ERR_UNSUPPORTED"
    assert bv(q_stride=[(1 << 22) + 128, 128, 1]) == "FA_ERR_UNSUPPORTED"
    assert bv(maxq=0, maxk=0) == "FA_OK"  # no rows and no keys: nothing launched
    assert bv(nb=1) == "FA_OK"  # B = 0
    assert bv(D=64, nb=1) == "FA_OK"
    # dS workspace sized by (sequences, Hq, max_seqlen_q, max_seqlen_k)
    assert bv(ds=T([3 * 4 * (256 * 64 + 4 * 64) - 1])) == "FA_ERR_SHAPE"
    assert bv(ds=T([3 * 4 * (256 * 64 + 4 * 64)], fa.FA_F16)) == "FA_ERR_DTYPE"
    assert bv(ds=T([1]), nb=1, maxq=0, maxk=0) == "FA_OK"  # B = 0: no dS to hold


def test_splitkv_default_count_follows_the_documented_rule(lib):
    # the header's rule, restated: ceil(256 / W) ranges (W = ceil(Sq / 256)
    # B Hq workgroups per range), at most max(1, Skv / 384) and 64, ranges
    # rounded up to multiples of 192 keys, those past the keys dropped
    rng = np.random.default_rng(5)
    for _ in range(400):
        B, Hq = int(rng.integers(1, 5)), int(rng.integers(1, 65))
        Sq, Skv = int(rng.integers(1, 3000)), int(rng.integers(1, 200000))
        W = -(-Sq // 256) * B * Hq
        ns = min(64, -(-256 // W), max(1, Skv // 384))
        length = -(-(-(-Skv // ns)) // 192) * 192
        want = -(-Skv // length)
        got = lib.fa_fwd_splitkv_splits(B, Hq, Sq, Skv, 0)
        assert got == want, (B, Hq, Sq, Skv, got, want)
        assert (got - 1) * length < Skv <= got * length


def test_splitkv_sizing_and_validation(lib):
    # sizing: ranges are multiples of 192 keys; the default fills the GPU
    assert lib.fa_fwd_splitkv_splits(1, 1, 100, 1000, 8) == 6   # 125 -> 192 keys per range
    assert lib.fa_fwd_splitkv_splits(1, 1, 100, 100, 8) == 1
    assert lib.fa_fwd_splitkv_splits(2, 16, 4096, 4096, 0) == 1  # already >= 256 workgroups
    assert lib.fa_fwd_splitkv_splits(1, 32, 512, 65536, 0) == 4  # 64 row blocks x 4 ranges fill 256 CUs once
    assert lib.fa_fwd_splitkv_splits(1, 32, 128, 32768, 0) == 8
    assert lib.fa_fwd_splitkv_splits(1, 1, 1, 1 << 20, 0) == 64
    assert lib.fa_fwd_splitkv_splits(1, 1, 1, 1000, 0) == 2     # at least 384 keys per range
    assert lib.fa_fwd_splitkv_splits(-1, 1, 1, 1, 0) == -1
    assert lib.fa_fwd_splitkv_workspace_elems(1, 32, 512, 65536, 128, 0) == 4 * 32 * 512 * 129
    assert lib.fa_fwd_splitkv_workspace_elems(1, 1, 100, 100, 128, 0) == 0
    q, k, v, o, lse = good(S=2000)

    def sk(ns=4, ws=T([4 * 2 * 4 * 2000 * 129], fa.FA_F32), q=q, k=k, v=v, o=o, causal=0):
        return name(lib, lib.fa_fwd_splitkv(R(q), R(k), R(v), None, None, causal, 0.1, 0.0, ns, R(ws), R(o), R(lse),
                                            None))

    assert sk(ns=65) == "FA_ERR_VALUE"
    assert sk(ns=-1) == "FA_ERR_VALUE"
    assert sk(ws=T([1000], fa.FA_F32)) == "FA_ERR_SHAPE"
    assert b"workspace holds" in lib.fa_last_error()
    assert sk(ws=T([4 * 2 * 4 * 2000 * 129], fa.FA_BF16)) == "FA_ERR_DTYPE"
    assert sk(ws=None) == "FA_ERR_NULL"
    q32, k32, v32, o32, l32 = good(S=2000, dt=fa.FA_F32)
    assert sk(q=q32, k=k32, v=v32, o=o32) == "FA_ERR_UNSUPPORTED"
    assert sk(causal=2) == "FA_ERR_VALUE"

    def na(ns=4, q=q, k=k, v=v, o=o):
        return name(lib, lib.fa_fwd_splitkv_noalloc(R(q), R(k), R(v), None, None, 0, 0.1, 0.0, ns, R(o), R(lse), None))

    # validation happens before the static scratch is looked up (no GPU here)
    assert na(ns=65) == "FA_ERR_VALUE"
    assert na(q=q32, k=k32, v=v32, o=o32) == "FA_ERR_UNSUPPORTED"
    big_q, big_k, big_v, big_o, big_l = good(B=2, Hq=32, Hkv=32, S=1024)
    kk = T([2, 32, 64 * 192, 128])
    assert name(lib, lib.fa_fwd_splitkv_noalloc(R(big_q), R(kk), R(kk), None, None, 0, 0.1, 0.0, 64, R(big_o),
                                                R(big_l), None)) == "FA_ERR_UNSUPPORTED"
    assert b"static scratch" in lib.fa_last_error()


def test_binding_refuses_cpu_tensors(lib):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors only"):
        fa.fa_fwd(q, q, q, scale=1.0)
    with pytest.raises(ValueError, match="GPU tensors only"):
        fa.fa_fwd_topk_gather(torch.zeros(1, 32, 576, dtype=torch.bfloat16),
                              torch.zeros(4, 576, dtype=torch.bfloat16),
                              torch.zeros(4, 512, dtype=torch.bfloat16),
                              torch.zeros(1, 4, dtype=torch.int32), scale=1.0)


def test_describe_marshals_shape_and_strides():
    t = torch.zeros(2, 3, 5, 8).transpose(1, 2)
    d = fa.describe(t)
    assert d.ndim == 4 and list(d.shape[:4]) == [2, 5, 3, 8] and list(d.stride[:4]) == [120, 8, 40, 1]
    assert d.dtype == fa.FA_F32
