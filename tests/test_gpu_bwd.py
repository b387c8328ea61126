"""GPU parity of fa_bwd (dense, causal, boolean mask, GQA; f16 / bf16, D = 128) against the
fp64 backward oracle, element by element, on seeded inputs.

Gate per gradient tensor (dq, dk, dv): the GPU path rounds P and dS to the
16-bit input type before the P^T dO, dS^T Q and dS K products and rounds the
results once more; each rounding has relative error at most u (2^-8 for bf16,
2^-11 for f16), and the errors are independent across the summed terms. The
relative L2 error of a gradient is then a small multiple of u; the gate allows
2.5 u, and every element must lie within 12 u of the largest reference
magnitude of its tensor (a term lost or doubled anywhere breaks both by orders
of magnitude)."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import gpu

pytestmark = pytest.mark.gpu

U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def _check(case, got, ref, dtype):
    g = got.float().cpu().numpy().astype(np.float64)
    err = g - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(err).max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    u = U[dtype]
    print("%s rel_l2 %.3e (gate %.3e) max_err/max_ref %.3e (gate %.3e)" % (case, rel, 2.5 * u, mx / max(scale, 1e-300), 12 * u))
    assert np.all(np.isfinite(g)), case
    assert rel <= 2.5 * u, (case, rel)
    assert mx <= 12 * u * scale, (case, mx, scale)


def run_bwd(case, B, Hq, Hkv, Sq, Skv, dtype, causal, seed, mask_fn=None):
    g0, q, k, v = synth.dense_inputs(seed, B, Hq, Hkv, Sq, Skv, 128, 128, dtype)
    mask = mask_fn(g0) if mask_fn else None
    g = synth.rng(seed + 1000)
    dout = synth.cast(synth.normal(g, (B, Hq, Sq, 128)), q.dtype)
    scale = 1 / math.sqrt(128)
    qg, kg, vg, dg = gpu(q, k, v, dout)
    mg = gpu(mask) if mask is not None else None
    o, lse = fa.fa_fwd(qg, kg, vg, scale=scale, causal=causal, mask=mg, rescale_threshold=0.0)
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=causal, mask=mg)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_dense_bwd(q, k, v, dout, scale=scale, causal=causal, mask=mask)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check("%s_%s" % (case, name), got, ref, q.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_gqa(dtype, causal):
    # 200 rows / keys: several 32-row tiles and a ragged tail in both
    # directions; two query heads per KV head.
    run_bwd("bwd_%s_causal%d" % (dtype, causal), 2, 4, 2, 200, 200, dtype, causal, 60 + causal)


@pytest.mark.parametrize("sq,skv", [(100, 300), (300, 100), (129, 129)])
def test_bwd_cross_lengths(sq, skv):
    # Sq < Skv, Sq > Skv (bottom-right causal: the first Sq - Skv rows see no
    # key and contribute nothing) and one row past a 128-row block.
    run_bwd("bwd_cross_%d_%d" % (sq, skv), 1, 2, 1, sq, skv, "bf16", True, 70 + sq)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_boolean_mask(dtype, causal):
    # [Sq, Skv] mask with 30% of the positions excluded (diagonal kept), on
    # the ragged GQA shape: excluded positions get P = 0 in both kernels.
    run_bwd("bwd_mask_%s_causal%d" % (dtype, causal), 2, 4, 2, 200, 200, dtype, causal, 90 + causal,
            mask_fn=lambda g: synth.bernoulli_mask(g, 200, 200, 0.3))


def test_bwd_mask_per_batch_with_empty_row():
    # [B, 1, Sq, Skv] mask (one per batch, broadcast over heads), Sq != Skv,
    # and one fully excluded row (LSE = -inf: it takes and gives no gradient).
    def m4(g):
        m = torch.from_numpy((g.random((2, 1, 150, 260)) < 0.2).astype(np.uint8))
        m[1, 0, 7] = 1
        return m
    run_bwd("bwd_mask4d", 2, 4, 2, 150, 260, "bf16", False, 95, mask_fn=m4)


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
        for name, got, ref in (("dq", dq[sl], rq), ("dk", dk[sl], rk), ("dv", dv[sl], rv)):
            _check("bwd_full_b%d_h%d_%s" % (b, h, name), got, ref, q.dtype)
