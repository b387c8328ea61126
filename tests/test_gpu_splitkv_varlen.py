"""GPU parity of fa_fwd_splitkv (key ranges + merge) and fa_fwd_varlen
(packed variable-length batches) against the fp64 oracle, on seeded inputs.

Both compute fa_fwd's attention: split-KV per (b, hq, i) row over the same
key set, the packed layout per sequence over its own rows and keys; the
oracle is the dense one (packed sequences are laid out into a padded
[B, H, maxlen, D] copy with per-batch lengths, a pure data move)."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import check, f32, gpu, sample_rows

pytestmark = pytest.mark.gpu


def run_split(case, q, k, v, scale, causal=False, sq=None, sk=None, num_splits=0, expect_splits=None):
    B, Hq, Sq, D = q.shape
    ns = fa.splitkv_splits(B, Hq, Sq, k.shape[2], num_splits)
    if expect_splits is not None:
        assert ns == expect_splits, ns
    o, lse = fa.fa_fwd_splitkv(*gpu(q, k, v), scale=scale, causal=causal, seqlens_q=gpu(sq), seqlens_k=gpu(sk),
                               num_splits=num_splits)
    torch.cuda.synchronize()
    kw = dict(scale=f32(scale), causal=causal, seqlens_q=sq, seqlens_k=sk)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), **kw)
    return check(case, o, lse, o_ref, lse_ref, q.dtype, o_abs, {"splits": ns})


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_splitkv_small(dtype, causal, D):
    # 100 rows over 3000 keys, 5 requested ranges -> 768-key ranges, 4 of them
    # (the last one ragged)
    _, q, k, v = synth.dense_inputs(600 + D + causal, 2, 4, 2, 100, 3000, D, D, dtype)
    run_split("splitkv_%s_D%d_causal%d" % (dtype, D, causal), q, k, v, 1 / math.sqrt(D), causal, num_splits=5,
              expect_splits=4)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Sq,Skv,expect", [(1, 1, 30000, 32), (2, 3, 20000, 15)])
def test_splitkv_decode_rows_default_ranges(B, Sq, Skv, expect, causal):
    # few query rows (decode-like) with the library's range count: 8 query
    # heads give 8 (16) workgroups per range, so 32 ranges of 960 keys (15 of
    # 1344, the last one ragged) put one workgroup on each of 256 CUs
    _, q, k, v = synth.dense_inputs(620 + Sq + causal, B, 8, 2, Sq, Skv, 128, 128, "bf16")
    run_split("splitkv_decode_B%d_Sq%d_causal%d" % (B, Sq, causal), q, k, v, 1 / math.sqrt(128), causal,
              expect_splits=expect)


def test_splitkv_lengths_and_empty_ranges():
    # per-batch lengths: batch 1 has 700 keys, so its ranges past them are
    # empty (LSE -inf, weight 0 in the merge); batch 2 has no rows at all
    _, q, k, v = synth.dense_inputs(610, 3, 4, 4, 64, 4000, 128, 128, "bf16")
    sq = torch.tensor([64, 50, 0], dtype=torch.int32)
    sk = torch.tensor([4000, 700, 900], dtype=torch.int32)
    rep = run_split("splitkv_lengths", q, k, v, 0.09, True, sq, sk, num_splits=8)
    assert rep["splits"] == 7  # 8 requested: 576-key ranges, 7 cover 4000 keys
    # a row whose keys all sit in one range and a causal row seeing no key
    _, q, k, v = synth.dense_inputs(611, 1, 2, 2, 300, 200, 128, 128, "f16")
    run_split("splitkv_sq_gt_skv", q, k, v, 0.09, True, num_splits=2)


def test_splitkv_matches_fa_fwd_and_single_range_is_fa_fwd():
    _, q, k, v = synth.dense_inputs(612, 1, 8, 2, 256, 5000, 128, 128, "bf16")
    qg, kg, vg = gpu(q, k, v)
    a, la = fa.fa_fwd(qg, kg, vg, scale=0.1, causal=True)
    b, lb = fa.fa_fwd_splitkv(qg, kg, vg, scale=0.1, causal=True)
    c, lc = fa.fa_fwd_splitkv(qg, kg, vg, scale=0.1, causal=True, num_splits=1)
    torch.cuda.synchronize()
    assert fa.splitkv_splits(1, 8, 256, 5000) > 1
    assert torch.equal(a, c) and torch.equal(la, lc)  # one range: the plain forward
    assert (la - lb).abs().max().item() < 2e-5
    # two results, each with its own P and output rounding (rel-L2 ~2e-3 from
    # the exact result): their difference is ~sqrt(2) times that
    diff = ((a.float() - b.float()).norm() / a.float().norm()).item()
    assert diff < 4e-3, diff


def test_full_splitkv_bf16_q512_k65536():
    w = synth.workload("splitkv_bf16_q512_k65536")
    q, k, v = w["q"], w["k"], w["v"]
    o, lse = fa.fa_fwd_splitkv(*gpu(q, k, v), scale=w["scale"], causal=True)
    torch.cuda.synchronize()
    B, Hq, Sq, D = q.shape
    rows = sample_rows(np.random.default_rng(55), B * Hq * Sq, 128, [0, Sq - 1, B * Hq * Sq - 1])
    kw = dict(scale=f32(w["scale"]), causal=True, rows=rows)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), **kw)
    idx = torch.from_numpy(rows).cuda()
    assert not torch.isnan(o).any() and torch.all(torch.isfinite(lse))
    check("full_splitkv_bf16_q512_k65536", o.reshape(-1, D)[idx], lse.reshape(-1)[idx], o_ref, lse_ref,
          torch.bfloat16, o_abs, {"sampled_rows": len(rows), "splits": fa.splitkv_splits(B, Hq, Sq, k.shape[2])},
          plain_cap=0.02)


# ---------------------------------------------------------------- packed varlen

def padded(x, cu, H, D, maxlen):
    """Packed [T, H, D] -> padded [B, H, maxlen, D] copy (zeros past each length)."""
    B = len(cu) - 1
    out = torch.zeros((B, H, maxlen, D), dtype=x.dtype)
    for b in range(B):
        n = int(cu[b + 1] - cu[b])
        out[b, :, :n] = x[int(cu[b]):int(cu[b + 1])].transpose(0, 1)
    return out


def varlen_reference(w, rows_per_seq=None, seed=0):
    """Oracle rows of a packed workload: for each sequence (a sample of) its
    rows; returns packed row ids (t * Hq + h), o_ref, lse_ref, o_abs."""
    q, k, v, cu_q, cu_k = w["q"], w["k"], w["v"], w["cu_q"].numpy(), w["cu_k"].numpy()
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    B = len(cu_q) - 1
    lq = np.diff(cu_q)
    lk = np.diff(cu_k)
    mq, mk = max(int(lq.max()), 1), max(int(lk.max()), 1)
    qp, kp, vp = padded(q, cu_q, Hq, D, mq), padded(k, cu_k, Hkv, D, mk), padded(v, cu_k, Hkv, D, mk)
    g = np.random.default_rng(seed)
    ids, packed = [], []
    for b in range(B):
        for h in range(Hq):
            n = int(lq[b])
            if n == 0:
                continue
            rs = np.arange(n) if rows_per_seq is None else np.unique(
                np.concatenate([g.choice(n, size=min(n, rows_per_seq), replace=False), [0, n - 1]]))
            ids.append((b * Hq + h) * mq + rs)
            packed.append((cu_q[b] + rs) * Hq + h)
    ids = np.concatenate(ids).astype(np.int64)
    packed = np.concatenate(packed).astype(np.int64)
    kw = dict(scale=f32(w["scale"]), causal=w["causal"], seqlens_q=torch.from_numpy(lq.astype(np.int32)),
              seqlens_k=torch.from_numpy(lk.astype(np.int32)), rows=ids)
    o_ref, lse_ref = oracle.attn_dense(qp, kp, vp, **kw)
    o_abs, _ = oracle.attn_dense(qp, kp, vp.abs(), **kw)
    return packed, o_ref, lse_ref, o_abs


def run_varlen(case, w, rows_per_seq=None, plain_cap=None):
    q, k, v = gpu(w["q"], w["k"], w["v"])
    Tq, Hq, D = q.shape
    o = torch.full((Tq + 5, Hq, D), 3.0, dtype=q.dtype, device="cuda")  # 5 rows outside every sequence
    lse = torch.full((Tq + 5, Hq), 3.0, dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, *gpu(w["cu_q"], w["cu_k"]), w["max_q"], scale=w["scale"], causal=w["causal"],
                     out=o[:Tq], lse=lse[:Tq])
    torch.cuda.synchronize()
    assert torch.all(o[Tq:] == 3.0) and torch.all(lse[Tq:] == 3.0)
    packed, o_ref, lse_ref, o_abs = varlen_reference(w, rows_per_seq)
    idx = torch.from_numpy(packed).cuda()
    return check(case, o[:Tq].reshape(-1, D)[idx], lse[:Tq].reshape(-1)[idx], o_ref, lse_ref, q.dtype, o_abs,
                 {"rows_checked": len(packed)}, plain_cap=plain_cap)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_varlen_small(causal, dtype):
    # lengths 300, 1, 0, 517 (a one-row sequence and an empty one), keys of
    # other lengths (Sq != Skv per sequence, bottom-right causal)
    w = synth.varlen(620 + causal, 4, 1, 600, 4, 2, 128, dtype=dtype, causal=causal, lens_q=[300, 1, 0, 517],
                     lens_k=[350, 40, 20, 517])
    assert w["max_q"] == 517
    run_varlen("varlen_%s_causal%d" % (dtype, causal), w)


def test_varlen_d64_gqa():
    w = synth.varlen(630, 5, 30, 400, 8, 2, 64, causal=True)
    run_varlen("varlen_d64_gqa", w)


def test_full_varlen_bf16_b16():
    w = synth.workload("varlen_bf16_b16")
    run_varlen("full_varlen_bf16_b16", w, rows_per_seq=12, plain_cap=0.02)
