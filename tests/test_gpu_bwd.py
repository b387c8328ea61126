"""GPU parity of fa_bwd and fa_bwd_varlen (dense, causal, boolean mask, GQA, packed batches; f16 /
bf16, D = 64 and 128) against the fp64 backward oracle, element by element, on seeded inputs, for
both dQ paths: from the dS the dK/dV kernel stores, and recomputing S and dP.

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
Below the 16-bit type's smallest normal number a rounding is off by up to
eta = half its smallest subnormal (2^-25 f16, 2^-134 bf16) instead, which adds
    eta (a + 1)
with a the sum of the magnitudes of what multiplies a rounded P or dS
(dV: dO over the rows, dK: scale Q over the rows, dQ: scale K over the keys;
f16's P of rarely seen keys lies there). rel-L2 per tensor <= u (measured
about 0.6 u). Gradients that must vanish (rows without keys, keys no row
sees) must be exactly 0."""
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
ETA = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}
LSE_REL = 1e-4


def underflow_scales(q, k, dout, scale):
    """a of the underflow term, per gradient, broadcast over rows / keys:
    dQ: scale sum_j |K_j|, dK: scale sum over the group's rows of |Q_i|,
    dV: the same sum of |dO_i| (shapes [B, H, 1, D])."""
    G = q.shape[1] // k.shape[1]
    sq = lambda x: np.abs(x.double().numpy()).sum(axis=2, keepdims=True)
    grp = lambda a: a.reshape(a.shape[0], -1, G, 1, a.shape[-1]).sum(axis=2)
    return scale * np.repeat(sq(k), G, axis=1), scale * grp(sq(q)), grp(sq(dout))


def _check(case, got, ref, bound, dtype, n_terms, under):
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    u = U[dtype]
    gate = (u + LSE_REL + n_terms * 2.0 ** -24) * bound + u * np.abs(ref) + ETA[dtype] * (under + 1.0)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float((err / gate).max()) if err.size else 0.0
    zero = bound == 0
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
    kw = dict(scale=scale, causal=causal, mask=mask, seqlens_q=sq, seqlens_k=sk)
    rq, rk, rv = oracle.attn_dense_bwd(q, k, v, dout, **kw)
    bq, bk, bv = oracle.attn_dense_bwd_bound(q, k, v, dout, **kw)
    G = Hq // Hkv
    aq, ak, av = underflow_scales(q, k, dout, scale)
    out = {}
    # both paths: dQ from the stored dS ("ds") and dQ recomputing S and dP
    for path, ws in (("ds", True), ("rc", None)):
        dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=causal, mask=mg, seqlens_q=sqg,
                               seqlens_k=skg, ds_workspace=ws)
        torch.cuda.synchronize()
        for name, got, ref, bnd, n, a in (("dq", dq, rq, bq, Skv, aq), ("dk", dk, rk, bk, G * Sq, ak),
                                          ("dv", dv, rv, bv, G * Sq, av)):
            _check("%s_%s_%s" % (case, path, name), got, ref, bnd, q.dtype, n, a)
        out[path] = (dq, dk, dv)
    assert torch.equal(out["ds"][2], out["rc"][2]), case  # dV does not depend on the path
    return out["ds"]


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
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, ds_workspace=True)
    dq1, dk1, dv1 = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, ds_workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(dv, dv1)
    # the two paths differ only by rounding (Delta's summation order, dQ's)
    for name, x, y in (("dq", dq, dq1), ("dk", dk, dk1)):
        r = float((x.float() - y.float()).norm() / y.float().norm())
        log("bwd_full_paths_" + name, {"rel_l2_between_paths": r})
        assert r <= 2.0 ** -8, (name, r)
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_dense_bwd(q[sl], k[sl], v[sl], dout[sl], scale=scale, causal=True)
        bq, bk, bv = oracle.attn_dense_bwd_bound(q[sl], k[sl], v[sl], dout[sl], scale=scale, causal=True)
        aq, ak, av = underflow_scales(q[sl], k[sl], dout[sl], scale)
        for name, got, ref, bnd, a in (("dq", dq[sl], rq, bq, aq), ("dk", dk[sl], rk, bk, ak),
                                       ("dv", dv[sl], rv, bv, av)):
            _check("bwd_full_b%d_h%d_%s" % (b, h, name), got, ref, bnd, q.dtype, S, a)


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


@pytest.mark.parametrize("ws", [True, None])
def test_bwd_precise_delta_from_o_lo(ws):
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
    dq0, dk0, dv0 = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, delta=d_plain, ds_workspace=ws)
    dq1, dk1, dv1 = fa.fa_bwd(qg, kg, vg, o, lse, dg, scale=scale, causal=True, o_lo=lo, delta=d_prec,
                              ds_workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dv0, dv1)  # dV does not use Delta
    o_ref, _ = oracle.attn_dense(q, k, v, scale=scale, causal=True)
    d_ref = (o_ref * dout.double().numpy()).sum(-1)
    e_plain = float(np.sqrt(np.mean((d_plain.cpu().double().numpy() - d_ref) ** 2)))
    e_prec = float(np.sqrt(np.mean((d_prec.cpu().double().numpy() - d_ref) ** 2)))
    rq, _, _ = oracle.attn_dense_bwd(q, k, v, dout, scale=scale, causal=True)
    r0 = float(np.linalg.norm(dq0.float().cpu().numpy() - rq) / np.linalg.norm(rq))
    r1 = float(np.linalg.norm(dq1.float().cpu().numpy() - rq) / np.linalg.norm(rq))
    log("bwd_precise_delta_%s" % ("ds" if ws else "rc"), {"delta_rms_err_plain": e_plain, "delta_rms_err_o_lo": e_prec,
                              "dq_rel_l2_plain": r0, "dq_rel_l2_o_lo": r1})
    assert e_prec < 0.75 * e_plain
    assert r1 < r0


# ---------------------------------------------------------------- packed varlen

def run_bwd_varlen(case, w, extra=3, o_lo_seed=None, ws=True):
    """fa_fwd_varlen then fa_bwd_varlen on a packed (TND) workload whose
    buffers carry `extra` trailing rows outside every sequence; each sequence
    is checked against the oracle's backward of that sequence alone (B = 1),
    Delta against its definition dO . (O + o_lo) in fp64 from the GPU's own O.
    Rows and keys outside every sequence must keep their prior contents.
    With o_lo_seed, a seeded o_lo (NaN on the rows outside every sequence)
    enters Delta; the gradients then leave the oracle's (which has no o_lo)
    and only Delta and dV (which does not use Delta) are checked."""
    q, k, v, cu_q, cu_k = w["q"], w["k"], w["v"], w["cu_q"], w["cu_k"]
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    G = Hq // Hkv
    lq, lk = np.diff(cu_q.numpy()), np.diff(cu_k.numpy())
    dout = synth.cast(synth.normal(synth.rng(w["seed"] + 1000), (Tq, Hq, D)), q.dtype)
    pad = lambda x: torch.cat([x, torch.ones((extra,) + tuple(x.shape[1:]), dtype=x.dtype)])
    qg, kg, vg, dg = gpu(pad(q), pad(k), pad(v), pad(dout))
    cqg, ckg = gpu(cu_q, cu_k)
    o = torch.full((Tq + extra, Hq, D), 5.0, dtype=q.dtype, device="cuda")
    lse = torch.full((Tq + extra, Hq), 5.0, dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(qg, kg, vg, cqg, ckg, w["max_q"], scale=w["scale"], causal=w["causal"],
                     rescale_threshold=0.0, out=o, lse=lse)
    lo = None
    if o_lo_seed is not None:
        lo = torch.full((Tq + extra, Hq, D), float("nan"), dtype=torch.float32)
        lo[:Tq] = torch.from_numpy(synth.normal(synth.rng(o_lo_seed), (Tq, Hq, D)) * np.float32(1e-3))
        lo = lo.cuda()
    sentinel = 7.0
    dq = torch.full((Tq + extra, Hq, D), sentinel, dtype=q.dtype, device="cuda")
    dk = torch.full((Tk + extra, Hkv, D), sentinel, dtype=q.dtype, device="cuda")
    dv = torch.full((Tk + extra, Hkv, D), sentinel, dtype=q.dtype, device="cuda")
    delta = torch.full((Tq + extra, Hq), sentinel, dtype=torch.float32, device="cuda")
    fa.fa_bwd_varlen(qg, kg, vg, cqg, ckg, w["max_q"], max(int(lk.max()), 1), o, lse, dg, scale=w["scale"],
                     causal=w["causal"], o_lo=lo, dq=dq, dk=dk, dv=dv, delta=delta, ds_workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(dq[Tq:] == sentinel) and torch.all(delta[Tq:] == sentinel)
    assert torch.all(dk[Tk:] == sentinel) and torch.all(dv[Tk:] == sentinel)
    for b in range(len(lq)):
        if lq[b] > 0 and lk[b] == 0:  # the forward of a sequence without keys: O = 0, LSE = -inf
            a0, a1 = int(cu_q[b]), int(cu_q[b + 1])
            assert torch.all(o[a0:a1] == 0) and torch.all(lse[a0:a1] == float("-inf")), case
    # Delta: an fp32 sum of the D products dO O (exact in fp32) and, with
    # o_lo, D more rounded ones: within 2 D 2^-24 of the sum of magnitudes.
    ov = o[:Tq].cpu().double()
    lv = lo[:Tq].cpu().double() if lo is not None else torch.zeros_like(ov)
    d_ref = (dout.double() * (ov + lv)).sum(-1)
    d_gate = 2 * D * 2.0 ** -24 * (dout.double().abs() * (ov.abs() + lv.abs())).sum(-1)
    d_err = (delta[:Tq].cpu().double() - d_ref).abs()
    log(case + "_delta", {"worst_ratio": float((d_err / (d_gate + 1e-300)).max())})
    assert torch.all(d_err <= d_gate), case
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    if lo is not None:
        return dq, dk, dv
    seq = lambda x, a, b: x[a:b].transpose(0, 1).unsqueeze(0).contiguous()
    for b in range(len(lq)):
        a0, a1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if a1 == a0 or k1 == k0:
            # no rows (its keys get dk = dv = 0) or no keys (its rows dq = 0)
            assert torch.all(dq[a0:a1] == 0) and torch.all(dk[k0:k1] == 0) and torch.all(dv[k0:k1] == 0)
            continue
        qs, ks, vs, ds = seq(q, a0, a1), seq(k, k0, k1), seq(v, k0, k1), seq(dout, a0, a1)
        kw = dict(scale=w["scale"], causal=w["causal"])
        rq, rk, rv = oracle.attn_dense_bwd(qs, ks, vs, ds, **kw)
        bq, bk, bv = oracle.attn_dense_bwd_bound(qs, ks, vs, ds, **kw)
        aq, ak, av = underflow_scales(qs, ks, ds, w["scale"])
        for name, got, ref, bnd, n, a in (("dq", seq(dq, a0, a1), rq, bq, k1 - k0, aq),
                                          ("dk", seq(dk, k0, k1), rk, bk, G * (a1 - a0), ak),
                                          ("dv", seq(dv, k0, k1), rv, bv, G * (a1 - a0), av)):
            _check("%s_seq%d_%s" % (case, b, name), got, ref, bnd, q.dtype, n, a)
    return dq, dk, dv


@pytest.mark.parametrize("ws", [True, None])
def test_bwd_varlen_tnd_fp16_causal(ws):
    # The packed TND case of the FlashAttentionScoreGrad pytest page (section
    # 5.4): four sequences of 114, 132, 14 and 287 tokens, 16 heads, D = 128,
    # fp16, causal; the gradients follow per sequence.
    w = synth.varlen(140, 4, 1, 300, 16, 16, 128, dtype="f16", causal=True, lens_q=[114, 132, 14, 287])
    w["seed"] = 140
    run_bwd_varlen("bwd_varlen_tnd06_%s" % ("ds" if ws else "rc"), w, ws=ws)


@pytest.mark.parametrize("ws", [True, None])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_gqa_cross_lengths(causal, ws):
    # bf16, two query heads per KV head, query and key lengths that differ
    # per sequence (bottom-right causal: the first rows of the 300 / 120
    # sequence see no key), a sequence without rows and a one-row sequence.
    w = synth.varlen(150 + causal, 5, 1, 300, 8, 4, 128, dtype="bf16", causal=causal,
                     lens_q=[300, 0, 1, 200, 77], lens_k=[120, 90, 40, 200, 260])
    w["seed"] = 150 + causal
    run_bwd_varlen("bwd_varlen_gqa_causal%d_%s" % (causal, "ds" if ws else "rc"), w, ws=ws)


@pytest.mark.parametrize("ws", [True, None])
def test_bwd_varlen_d64_keyless_sequence_and_o_lo(ws):
    # D = 64 (its own swizzle and copy split) with a sequence that has rows
    # but no keys (LSE = -inf: dq = 0 there); then Delta read through a
    # seeded o_lo at the packed offsets (dV, which does not use Delta, must
    # not change).
    w = synth.varlen(160, 4, 1, 300, 4, 2, 64, dtype="f16", causal=False, lens_q=[150, 40, 233, 9],
                     lens_k=[170, 0, 100, 64])
    w["seed"] = 160
    tag = "ds" if ws else "rc"
    _, _, dv0 = run_bwd_varlen("bwd_varlen_d64_" + tag, w, ws=ws)
    _, _, dv1 = run_bwd_varlen("bwd_varlen_d64_o_lo_" + tag, w, o_lo_seed=161, ws=ws)
    assert torch.equal(dv0, dv1)
