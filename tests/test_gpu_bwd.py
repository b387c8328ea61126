"""GPU parity of fa_bwd (dense, causal, boolean mask, GQA; f16 / bf16, D = 64 and 128) against the
fp64 backward oracle, element by element, on seeded inputs.

Per-element gate (no page states one for the backward; derived here): the GPU
path rounds P to the 16-bit input type before dV = P^T dO, rounds dS before
dK = scale dS^T Q and dQ = scale dS K, forms Delta_i = dO_i . O_i from the
forward's rounded O, recomputes P from the forward's fp32 LSE, and rounds
each gradient once more. With unit roundoff u (2^-8 bf16, 2^-11 f16) every
element then lies within
    (u + 1e-4 + n 2^-24) g + u |ref|
of the exact gradient, where g is the oracle's first-order error scale of that
element (the sum of the magnitudes of the terms the GPU rounds, with the
Delta error of the forward's rounded O folded in: oracle.attn_dense_bwd_bound),
1e-4 the forward's LSE tolerance (a relative error of the recomputed P), n the
number of summed terms (fp32 accumulation) and u |ref| the final rounding.
rel-L2 per tensor <= u (measured about 0.6 u). Gradients that must vanish
(rows without keys, keys no row sees) must be exactly 0."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import gpu, log

pytestmark = pytest.mark.gpu

U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
LSE_REL = 1e-4


def _check(case, got, ref, bound, dtype, n_terms):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    u = U[dtype]
    gate = (u + LSE_REL + n_terms * 2.0 ** -24) * bound + u * np.abs(ref)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float((err / np.where(gate > 0, gate, 1.0)).max()) if err.size else 0.0
    zero = gate == 0
    log(case, {"rel_l2": rel, "rel_l2_over_u": rel / u, "worst_ratio": worst,
               "n_forced_zero": int(zero.sum())})
    assert np.all(np.isfinite(g)), case
    assert rel <= u, (case, rel)
    assert np.all(err <= gate), (case, worst)
    assert np.all(g[zero] == 0.0), case


def run_bwd(case, B, Hq, Hkv, Sq, Skv, dtype, causal, seed, mask_fn=None, sq=None, sk=None, D=128):
    g0, q, k, v = synth.dense_inputs(seed, B, Hq, Hkv, Sq, Skv, D, D, dtype)
    mask = mask_fn(g0) if mask_fn else None
    g = synth.rng(seed + 1000)
    dout = synth.cast(synth.normal(g, (B, Hq, Sq, D)), q.dtype)
    scale = 1 / math.sqrt(D)
    qg, kg, vg, dg, mg = gpu(q, k, v, dout, mask)
    sqg, skg = gpu(sq, sk)
    o, lse = fa.fa_fwd(qg, kg, vg, scale=scale, causal=causal, mask=mg, seqlens_q=sqg, seqlens_k=skg)
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=causal, mask=mg, seqlens_q=sqg,
                           seqlens_k=skg)
    torch.cuda.synchronize()
    kw = dict(scale=scale, causal=causal, mask=mask, seqlens_q=sq, seqlens_k=sk)
    rq, rk, rv = oracle.attn_dense_bwd(q, k, v, dout, **kw)
    bq, bk, bv = oracle.attn_dense_bwd_bound(q, k, v, dout, **kw)
    G = Hq // Hkv
    for name, got, ref, bnd, n in (("dq", dq, rq, bq, Skv), ("dk", dk, rk, bk, G * Sq), ("dv", dv, rv, bv, G * Sq)):
        _check("%s_%s" % (case, name), got, ref, bnd, q.dtype, n)
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_gqa(dtype, causal):
    # 200 rows / keys: several 32-row tiles and a ragged tail in both
    # directions; two query heads per KV head.
    run_bwd("bwd_%s_causal%d" % (dtype, causal), 2, 4, 2, 200, 200, dtype, causal, 60 + causal)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_head_dim_64(dtype, causal):
    # D = 64: its own tile swizzle and copy split; ragged rows and keys, two
    # query heads per KV head, Sq != Skv.
    run_bwd("bwd_d64_%s_causal%d" % (dtype, causal), 2, 4, 2, 170, 230, dtype, causal, 110 + causal, D=64)


def test_bwd_head_dim_64_mask_and_lengths():
    # D = 64 with a per-head boolean mask and per-batch lengths (padded rows
    # and keys get exact zeros).
    sq = torch.tensor([150, 61], dtype=torch.int32)
    sk = torch.tensor([140, 200], dtype=torch.int32)

    def mh(g):
        return torch.from_numpy((g.random((1, 4, 150, 200)) < np.array([0.2, 0.4, 0.1, 0.6])[None, :, None, None])
                                .astype(np.uint8))
    dq, dk, dv = run_bwd("bwd_d64_mask_lengths", 2, 4, 2, 150, 200, "bf16", True, 113, mask_fn=mh, sq=sq, sk=sk,
                         D=64)
    assert torch.all(dq[1, :, 61:] == 0) and torch.all(dk[0, :, 140:] == 0) and torch.all(dv[0, :, 140:] == 0)


@pytest.mark.parametrize("sq,skv", [(100, 300), (300, 100), (129, 129)])
def test_bwd_cross_lengths(sq, skv):
    # Sq < Skv, Sq > Skv (bottom-right causal: the first Sq - Skv rows see no
    # key and contribute nothing) and one row past a 128-row block.
    dq, _, _ = run_bwd("bwd_cross_%d_%d" % (sq, skv), 1, 2, 1, sq, skv, "bf16", True, 70 + sq)
    if sq > skv:
        assert torch.all(dq[:, :, :sq - skv] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_boolean_mask(dtype, causal):
    # [Sq, Skv] mask with 30% of the positions excluded (diagonal kept), on
    # the ragged GQA shape: excluded positions get P = 0 in both kernels.
    run_bwd("bwd_mask_%s_causal%d" % (dtype, causal), 2, 4, 2, 200, 200, dtype, causal, 90 + causal,
            mask_fn=lambda g: synth.bernoulli_mask(g, 200, 200, 0.3))


def test_bwd_mask_per_batch_with_empty_row_and_column():
    # [B, 1, Sq, Skv] mask (one per batch, broadcast over heads), Sq != Skv,
    # one fully excluded row (LSE = -inf: it takes and gives no gradient) and
    # one fully excluded key (no row sees it: dK = dV = 0 there).
    def m4(g):
        m = torch.from_numpy((g.random((2, 1, 150, 260)) < 0.2).astype(np.uint8))
        m[1, 0, 7] = 1
        m[0, 0, :, 33] = 1
        return m
    dq, dk, dv = run_bwd("bwd_mask4d", 2, 4, 2, 150, 260, "bf16", False, 95, mask_fn=m4)
    assert torch.all(dq[1, :, 7] == 0)
    assert torch.all(dk[0, :, 33] == 0) and torch.all(dv[0, :, 33] == 0)


def test_bwd_mask_per_head_causal_cross_lengths():
    # [1, Hq, Sq, Skv] mask that differs per query head, two query heads per
    # KV head, causal with Sq != Skv: a wrong query-head offset into the mask
    # in either gradient kernel reads another head's bytes.
    def mh(g):
        return torch.from_numpy((g.random((1, 4, 170, 230)) < np.array([0.1, 0.5, 0.3, 0.7])[None, :, None, None])
                                .astype(np.uint8))
    run_bwd("bwd_mask_per_head", 2, 4, 2, 170, 230, "f16", True, 96, mask_fn=mh)


def test_bwd_full_size_heads_sampled():
    # The causal bf16 B=2, H=16, S=4096 workload: the kernels run on the whole
    # problem; two (batch, head) slices are checked against the oracle.
    B, H, S = 2, 16, 4096
    _, q, k, v = synth.dense_inputs(80, B, H, H, S, S, 128, 128, "bf16")
    g = synth.rng(1080)
    dout = synth.cast(synth.normal(g, (B, H, S, 128)), q.dtype)
    scale = 1 / math.sqrt(128)
    qg, kg, vg, dg = gpu(q, k, v, dout)
    o, lse = fa.fa_fwd(qg, kg, vg, scale=scale, causal=True, rescale_threshold=0.0)
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_dense_bwd(q[sl], k[sl], v[sl], dout[sl], scale=scale, causal=True)
        bq, bk, bv = oracle.attn_dense_bwd_bound(q[sl], k[sl], v[sl], dout[sl], scale=scale, causal=True)
        for name, got, ref, bnd in (("dq", dq[sl], rq, bq), ("dk", dk[sl], rk, bk), ("dv", dv[sl], rv, bv)):
            _check("bwd_full_b%d_h%d_%s" % (b, h, name), got, ref, bnd, q.dtype, S)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sequence_lengths(causal):
    # Per-batch lengths: padded rows take part in nothing and get dq = 0,
    # padded keys get dk = dv = 0 (the gate forces exact zeros wherever the
    # oracle's error scale is 0); a batch with no rows at all.
    sq = torch.tensor([200, 77, 0], dtype=torch.int32)
    sk = torch.tensor([200, 150, 10], dtype=torch.int32)
    dq, dk, dv = run_bwd("bwd_seqlens_causal%d" % causal, 3, 4, 2, 200, 200, "bf16", causal, 97 + causal,
                         sq=sq, sk=sk)
    assert torch.all(dq[1, :, 77:] == 0) and torch.all(dq[2] == 0)
    assert torch.all(dk[1, :, 150:] == 0) and torch.all(dv[2] == 0) and torch.all(dk[2] == 0)


def test_bwd_precise_delta_from_o_lo():
    # Delta = dO . (o + o_lo) instead of dO . o: the forward's output rounding
    # no longer enters Delta (the precise dpsum of the sparse-MLA page). Peaked
    # rows (q scaled up) make Delta's error matter for dQ.
    B, H, S = 1, 4, 256
    g0, q, k, v = synth.dense_inputs(98, B, H, H, S, S, 128, 128, "bf16")
    q = (q.float() * 4.0).to(torch.bfloat16)
    dout = synth.cast(synth.normal(synth.rng(1098), (B, H, S, 128)), q.dtype)
    scale = 1 / math.sqrt(128)
    qg, kg, vg, dg = gpu(q, k, v, dout)
    o, lse, lo = fa.fa_fwd(qg, kg, vg, scale=scale, causal=True, return_o_lo=True)
    d_plain = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    d_prec = torch.empty_like(d_plain)
    dq0, dk0, dv0 = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, delta=d_plain)
    dq1, dk1, dv1 = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, o_lo=lo, delta=d_prec)
    torch.cuda.synchronize()
    assert torch.equal(dv0, dv1)  # dV does not use Delta
    o_ref, _ = oracle.attn_dense(q, k, v, scale=scale, causal=True)
    d_ref = (o_ref * dout.double().numpy()).sum(-1)
    e_plain = float(np.sqrt(np.mean((d_plain.cpu().double().numpy() - d_ref) ** 2)))
    e_prec = float(np.sqrt(np.mean((d_prec.cpu().double().numpy() - d_ref) ** 2)))
    rq, _, _ = oracle.attn_dense_bwd(q, k, v, dout, scale=scale, causal=True)
    r0 = float(np.linalg.norm(dq0.float().cpu().numpy() - rq) / np.linalg.norm(rq))
    r1 = float(np.linalg.norm(dq1.float().cpu().numpy() - rq) / np.linalg.norm(rq))
    log("bwd_precise_delta", {"delta_rms_err_plain": e_plain, "delta_rms_err_o_lo": e_prec,
                              "dq_rel_l2_plain": r0, "dq_rel_l2_o_lo": r1})
    assert e_prec < 0.75 * e_plain
    assert r1 < r0
