"""GPU parity of fa_fwd (dense, causal, boolean mask, GQA, sequence lengths)
against the fp64 oracle, element by element, on seeded inputs."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import absv, check, f32, gpu, log, sample_rows
from oracle import metrics

pytestmark = pytest.mark.gpu


def run_dense(case, q, k, v, scale, causal=False, mask=None, sq=None, sk=None, thr=0.0):
    o, lse = fa.fa_fwd(*gpu(q, k, v), scale=scale, causal=causal, mask=gpu(mask),
                       seqlens_q=gpu(sq), seqlens_k=gpu(sk), rescale_threshold=thr)
    torch.cuda.synchronize()
    kw = dict(scale=f32(scale), causal=causal, mask=mask, seqlens_q=sq, seqlens_k=sk)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, absv(v), **kw)
    return check(case, o, lse, o_ref, lse_ref, q.dtype, o_abs)


@pytest.mark.parametrize("thr", [0.0, 8.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_ragged(dtype, D, causal, thr):
    # 300 rows/keys: several 64-key tiles, a ragged tail, a partial query block;
    # thr 0 = exact running max, 8 = lazy rescale
    _, q, k, v = synth.dense_inputs(100 + D + causal, 2, 4, 4, 300, 300, D, D, dtype)
    run_dense("dense_%s_D%d_causal%d_thr%g" % (dtype, D, causal, thr), q, k, v, 1 / math.sqrt(D), causal,
              thr=thr)


@pytest.mark.parametrize("skv", [95, 96, 97, 191, 192, 193])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_boundaries_d128(skv, causal):
    # Key counts around the 96-key tiles of the D = 128 kernels (one key short
    # of, exactly at and one past a tile edge), queries over two workgroups.
    dtype = "f16" if skv % 2 else "bf16"
    _, q, k, v = synth.dense_inputs(300 + skv + causal, 1, 2, 2, 300, skv, 128, 128, dtype)
    run_dense("tiles_skv%d_causal%d" % (skv, causal), q, k, v, 1 / math.sqrt(128), causal, thr=0.0)
    _, q, k, v = synth.dense_inputs(400 + skv + causal, 1, 2, 2, skv, skv, 128, 128, dtype)
    run_dense("tiles_sq_skv%d_causal%d" % (skv, causal), q, k, v, 1 / math.sqrt(128), causal, thr=8.0)


@pytest.mark.parametrize("thr", [0.0, 8.0])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gqa_causal_mask(dtype, thr):
    g, q, k, v = synth.dense_inputs(7, 2, 8, 2, 333, 333, 128, 128, dtype)
    mask = synth.bernoulli_mask(g, 333, 333, 0.05)
    run_dense("gqa_mask_%s_thr%g" % (dtype, thr), q, k, v, 1 / math.sqrt(128), True, mask, thr=thr)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_mask_gqa(D, causal):
    # The fp32 kernel with a boolean mask that differs per query head
    # ([1, Hq, Sq, Skv]), two query heads per KV head, Sq != Skv (bottom-right
    # causal) and a ragged tail in both directions.
    g, q, k, v = synth.dense_inputs(40 + causal + D, 1, 4, 2, 150, 230, D, D, "f32")
    dens = np.array([0.05, 0.3, 0.15, 0.6])[None, :, None, None]
    m = torch.from_numpy((g.random((1, 4, 150, 230)) < dens).astype(np.uint8))
    run_dense("f32_mask_gqa_d%d_causal%d" % (D, causal), q, k, v, 1 / math.sqrt(D), causal, m)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_head_groups_unequal_lengths(causal):
    # Eight (batch, KV head) pairs and two query heads per KV head: the work
    # decode gives the two head groups different pair orders; the batches
    # have different lengths.
    _, q, k, v = synth.dense_inputs(12 + causal, 2, 8, 4, 300, 300, 128, 128, "bf16")
    sl = torch.tensor([300, 170], dtype=torch.int32)
    run_dense("gqa_groups_causal%d" % causal, q, k, v, 1 / math.sqrt(128), causal, None, sl, sl)


@pytest.mark.parametrize("causal", [False, True])
def test_mask_aligned_rows(causal):
    # Mask rows 16-byte aligned (Skv = 336): full 64-key tiles take the
    # coalesced 16-byte mask loads, the partial last tile the byte loads.
    g, q, k, v = synth.dense_inputs(17 + causal, 2, 4, 2, 300, 336, 128, 128, "f16")
    mask = synth.bernoulli_mask(g, 300, 336, 0.3)
    run_dense("mask_aligned_causal%d" % causal, q, k, v, 1 / math.sqrt(128), causal, mask, thr=0.0)
    m4 = torch.from_numpy((g.random((2, 1, 300, 336)) < 0.2).astype(np.uint8))
    m4[1, 0, 7] = 1  # a fully masked row
    run_dense("mask4d_aligned_causal%d" % causal, q, k, v, 1 / math.sqrt(128), causal, m4, thr=8.0)


def _mask_view(mask_dev, pad):
    """The same mask bytes in storage whose rows are `pad` bytes longer, so
    that rows are no longer 16-byte chunks (pad 1: byte loads, pad 4: 4-byte
    loads into registers)."""
    *lead, sq, skv = mask_dev.shape
    big = torch.ones(*lead, sq, skv + pad, dtype=torch.uint8, device=mask_dev.device)
    big[..., :skv] = mask_dev
    return big[..., :skv]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_mask_lds_staged(D, causal):
    # Masks whose rows are whole 16-byte chunks are staged through LDS with
    # the K/V tiles (permuted key order inside each 32-key half); any other
    # mask goes through registers. Both must match the oracle, with per-batch
    # lengths, Sq != Skv (rows without keys under the causal mask), a partial
    # last tile, rows past Sq in the last workgroup, a fully masked row and
    # per-head masks broadcast over the batch.
    g, q, k, v = synth.dense_inputs(31 + D + causal, 2, 4, 2, 290, 272, D, D, "f16")
    m = torch.from_numpy((g.random((1, 4, 290, 272)) < 0.25).astype(np.uint8))
    m[0, 2, 11] = 1
    sq = torch.tensor([290, 203], dtype=torch.int32)
    sk = torch.tensor([272, 144], dtype=torch.int32)
    scale = 1 / math.sqrt(D)
    run_dense("mask_lds_D%d_causal%d" % (D, causal), q, k, v, scale, causal, m, sq, sk)
    qg, kg, vg, mg, sqg, skg = gpu(q, k, v, m, sq, sk)
    outs = []
    for pad in (0, 1, 4):
        mm = mg if pad == 0 else _mask_view(mg, pad)
        outs.append(fa.fa_fwd(qg, kg, vg, scale=scale, causal=causal, mask=mm, seqlens_q=sqg, seqlens_k=skg))
    torch.cuda.synchronize()
    kw = dict(scale=f32(scale), causal=causal, mask=m, seqlens_q=sq, seqlens_k=sk)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, absv(v), **kw)
    for pad, (o, lse) in zip((0, 1, 4), outs):
        check("mask_lds_D%d_causal%d_pad%d" % (D, causal, pad), o, lse, o_ref, lse_ref, q.dtype, o_abs)
    # LDS-staged and register paths sum the keys of a half in different
    # orders: they agree to rounding, and exactly on rows without keys.
    (o0, l0), (o1, l1) = outs[0], outs[1]
    assert (o0.float() - o1.float()).abs().max().item() <= 2 ** -9 * max(1.0, o1.float().abs().max().item())
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l0))
    assert (l0[fin] - l1[fin]).abs().max().item() <= 1e-5


def test_growing_scores_rescale_paths():
    # Scores that keep growing along the keys force a rescale on every tile
    # with the exact max and on some tiles with the lazy one; both must match.
    g, q, k, v = synth.dense_inputs(21, 1, 2, 2, 256, 640, 128, 128, "bf16")
    ramp = torch.linspace(0.2, 3.0, 640).view(1, 1, 640, 1)
    k = (k.float() * ramp).to(k.dtype)
    for thr in (0.0, 2.0, 8.0):
        run_dense("ramp_thr%g" % thr, q, k, v, 1 / math.sqrt(128), False, thr=thr)


def test_mask_4d_broadcasts_and_empty_rows():
    g, q, k, v = synth.dense_inputs(8, 2, 3, 1, 130, 200, 64, 64, "f16")
    m = torch.from_numpy((g.random((2, 1, 130, 200)) < 0.3).astype(np.uint8))
    m[1, 0, 5] = 1  # a fully masked row -> O = 0, LSE = -inf
    rep = run_dense("mask4d_b1", q, k, v, 0.125, False, m)
    m2 = torch.from_numpy((g.random((1, 3, 130, 200)) < 0.5).astype(np.uint8))
    run_dense("mask4d_1h", q, k, v, 0.125, True, m2)
    assert rep["rows"] == 2 * 3 * 130


def test_zero_mask_matches_no_mask():
    # An all-zero boolean mask excludes nothing. The masked and unmasked
    # D = 128 kernels tile the keys differently (64 and 96 keys), so the two
    # results agree to rounding, and each matches the oracle.
    _, q, k, v = synth.dense_inputs(9, 1, 2, 2, 190, 190, 128, 128, "bf16")
    zero = torch.zeros((190, 190), dtype=torch.uint8)
    run_dense("zero_mask", q, k, v, 0.1, True, zero)
    qq, kk, vv = gpu(q, k, v)
    a, la = fa.fa_fwd(qq, kk, vv, scale=0.1, causal=True)
    b, lb = fa.fa_fwd(qq, kk, vv, scale=0.1, causal=True, mask=zero.cuda())
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 2 ** -7 * max(1.0, a.float().abs().max().item())
    assert (la - lb).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_seqlens_and_cross_lengths(dtype):
    _, q, k, v = synth.dense_inputs(10, 3, 2, 2, 257, 400, 128, 128, dtype)
    sq = torch.tensor([257, 100, 0], dtype=torch.int32)
    sk = torch.tensor([400, 77, 5], dtype=torch.int32)
    run_dense("seqlens_causal_%s" % dtype, q, k, v, 0.09, True, None, sq, sk)
    run_dense("seqlens_%s" % dtype, q, k, v, 0.09, False, None, sq, sk)
    run_dense("cross_causal_%s" % dtype, q[:, :, :100], k, v, 0.09, True)  # Sq < Skv


def test_strided_bsnd_views():
    g = synth.rng(11)
    q = synth.cast(synth.normal(g, (2, 150, 4, 128)), torch.bfloat16)  # [B, S, H, D]
    k = synth.cast(synth.normal(g, (2, 150, 4, 128)), torch.bfloat16)
    v = synth.cast(synth.normal(g, (2, 150, 4, 128)), torch.bfloat16)
    qg, kg, vg = (t.cuda().transpose(1, 2) for t in (q, k, v))  # BNSD views, not contiguous
    o, lse = fa.fa_fwd(qg, kg, vg, scale=0.088, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_dense(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                       scale=f32(0.088), causal=True)
    o_abs, _ = oracle.attn_dense(q.transpose(1, 2), k.transpose(1, 2), v.abs().transpose(1, 2),
                                 scale=f32(0.088), causal=True)
    check("strided_bsnd", o, lse, o_ref, lse_ref, torch.bfloat16, o_abs)


def test_out_of_range_memory_is_never_read():
    # K/V rows past Skv (and past seqlens_k) hold NaN: they must not leak.
    _, q, k, v = synth.dense_inputs(12, 1, 2, 2, 100, 100, 128, 128, "f16")
    kp = torch.full((1, 2, 164, 128), float("nan"), dtype=torch.float16, device="cuda")
    vp = torch.full((1, 2, 164, 128), float("nan"), dtype=torch.float16, device="cuda")
    kp[:, :, :100] = k.cuda()
    vp[:, :, :100] = v.cuda()
    o, lse = fa.fa_fwd(q.cuda(), kp[:, :, :100], vp[:, :, :100], scale=0.1, causal=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=f32(0.1))
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), scale=f32(0.1))
    check("nan_tail", o, lse, o_ref, lse_ref, torch.float16, o_abs)
    kp[:, :, 60:100] = float("nan")
    vp[:, :, 60:100] = float("nan")
    sk = torch.tensor([60], dtype=torch.int32)
    o, lse = fa.fa_fwd(q.cuda(), kp[:, :, :100], vp[:, :, :100], scale=0.1, seqlens_k=sk.cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=f32(0.1), seqlens_k=sk)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), scale=f32(0.1), seqlens_k=sk)
    check("nan_past_seqlen", o, lse, o_ref, lse_ref, torch.float16, o_abs)


def test_extreme_rows_fp16():
    g, q, k, v = synth.dense_inputs(13, 1, 4, 4, 256, 256, 128, 128, "f16")
    q32 = q.float()
    q32[0, 1, ::7] *= 30.0
    q = q32.half()
    run_dense("extreme_x30_f16", q, k, v, 1 / math.sqrt(128), True)


def test_single_key_and_single_row():
    _, q, k, v = synth.dense_inputs(14, 1, 1, 1, 1, 1, 128, 128, "bf16")
    o, lse = fa.fa_fwd(*gpu(q, k, v), scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), v)  # one key: O = V exactly
    _, q, k, v = synth.dense_inputs(15, 1, 1, 1, 64, 64, 64, 64, "f32")
    o, _ = fa.fa_fwd(*gpu(q, k, v), scale=0.3, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu()[0, 0, 0], v[0, 0, 0])  # first causal row sees key 0 only


def test_default_is_exact_running_max():
    # The binding's default rescale threshold is 0: the exact running max.
    _, q, k, v = synth.dense_inputs(18, 1, 2, 2, 300, 300, 128, 128, "bf16")
    qq, kk, vv = gpu(q, k, v)
    a, la = fa.fa_fwd(qq, kk, vv, scale=0.1, causal=True)
    b, lb = fa.fa_fwd(qq, kk, vv, scale=0.1, causal=True, rescale_threshold=0.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_empty_problems():
    _, q, k, v = synth.dense_inputs(16, 1, 2, 2, 8, 8, 64, 64, "bf16")
    qq, kk, vv = gpu(q, k, v)
    o, lse = fa.fa_fwd(qq[:, :, :0], kk, vv, scale=1.0)  # Sq = 0
    assert o.shape == (1, 2, 0, 64)
    o, lse = fa.fa_fwd(qq, kk[:, :, :0], vv[:, :, :0], scale=1.0)  # Skv = 0
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    o, lse = fa.fa_fwd(qq[:0], kk[:0], vv[:0], scale=1.0)  # B = 0
    assert o.shape == (0, 2, 8, 64)


# ---------------------------------------------------------------------------
# Full-size workloads, checked on sampled rows computed one by one by the
# oracle, in the launch configuration the benchmark times: the exact running
# max (rescale threshold 0, the contract path) and the lazy rescale
# (threshold 8) on the same inputs.
# ---------------------------------------------------------------------------

def _full_dense(name, n_rows, must_rows=(), plain_cap=None, page_gate=False):
    w = synth.workload(name)
    q, k, v = w["q"], w["k"], w["v"]
    mask = w.get("mask")
    qg, kg, vg, mg = gpu(q, k, v, mask)
    B, Hq, Sq, D = q.shape
    g = np.random.default_rng(1234)
    must = list(must_rows)
    if "scaled_rows" in w:
        must += list(g.choice(w["scaled_rows"].numpy(), size=64, replace=False))
    rows = sample_rows(g, B * Hq * Sq, n_rows, must + [0, B * Hq * Sq - 1, Sq - 1, Sq])
    kw = dict(scale=f32(w["scale"]), causal=w["causal"], mask=mask, rows=rows)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), **kw)
    idx = torch.from_numpy(rows).cuda()
    reps = {}
    for thr in (0.0, 8.0):
        o, lse = fa.fa_fwd(qg, kg, vg, scale=w["scale"], causal=w["causal"], mask=mg, rescale_threshold=thr)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        assert torch.all(torch.isfinite(lse))  # every row of these workloads has a key
        reps[thr] = check("full_%s_thr%g" % (name, thr), o.reshape(-1, D)[idx], lse.reshape(-1)[idx], o_ref,
                          lse_ref, q.dtype, o_abs, {"sampled_rows": len(rows), "rescale_threshold": thr},
                          plain_cap=plain_cap, page_gate=page_gate)
        del o, lse
    return reps


def test_full_dense_f32_s128():
    w = synth.workload("dense_f32_s128")
    o_ref, lse_ref = oracle.attn_dense(w["q"], w["k"], w["v"], scale=f32(w["scale"]))
    o_abs, _ = oracle.attn_dense(w["q"], w["k"], w["v"].abs(), scale=f32(w["scale"]))
    for thr in (0.0, 8.0):
        o, lse = fa.fa_fwd(*gpu(w["q"], w["k"], w["v"]), scale=w["scale"], rescale_threshold=thr)
        torch.cuda.synchronize()
        check("full_dense_f32_s128_thr%g" % thr, o, lse, o_ref, lse_ref, torch.float32, o_abs)


def test_full_causal_bf16_s4096():
    _full_dense("causal_bf16_s4096", 384, plain_cap=0.02)


def test_full_causal_bf16_s8192():
    _full_dense("causal_bf16_s8192", 256, plain_cap=0.02)


def test_full_gqa_mask_f16_s8192():
    # fp16 at full size: the literal atol/rtol gate on every sampled element
    _full_dense("gqa_mask_f16_s8192", 256, plain_cap=0.0, page_gate=True)


# ---------------------------------------------------------------------------
# The o_lo output: fp32(O) - rounded(O), the output's rounding residual.
# ---------------------------------------------------------------------------

def check_o_lo(case, o, lo, o_ref, o_abs, dtype, n_keys):
    """o + o_lo is the unrounded fp32 result: rounding it reproduces o bit for
    bit, |o_lo| is at most half an ulp of o, and it lies within the error of
    rounding P alone (no output-rounding term: u_P sum_j P_j |v_j| plus fp32
    accumulation) of the oracle, which o itself does not."""
    x = o.float() + lo
    assert torch.equal(x.to(o.dtype), o), case
    # half an ulp: relative 2^-8 (bf16) / 2^-11 (fp16), absolute 2^-25 for
    # fp16's subnormal range
    u_out = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    sub = 0.0 if dtype == torch.bfloat16 else 2.0 ** -25
    assert torch.all(lo.abs() <= u_out * (1 + 2 * u_out) * o.float().abs() + sub), case
    xn = x.cpu().numpy().astype(np.float64)
    on = o.float().cpu().numpy().astype(np.float64)
    o_ref = np.asarray(o_ref).reshape(xn.shape)
    o_abs = np.asarray(o_abs).reshape(xn.shape)
    u_p = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    gate = (u_p + n_keys * 2.0 ** -24 + 1e-4) * o_abs + 1e-6
    err_x = np.abs(xn - o_ref)
    rx, ro = metrics.rel_l2(xn, o_ref), metrics.rel_l2(on, o_ref)
    log(case, {"rel_l2_o": ro, "rel_l2_o_plus_o_lo": rx, "worst_ratio": float((err_x / gate).max())})
    assert np.all(err_x <= gate), case
    assert rx < ro, case


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_o_lo_dense(dtype, causal):
    _, q, k, v = synth.dense_inputs(500 + causal, 2, 4, 2, 300, 300, 128, 128, dtype)
    o, lse, lo = fa.fa_fwd(*gpu(q, k, v), scale=0.088, causal=causal, return_o_lo=True)
    a, la = fa.fa_fwd(*gpu(q, k, v), scale=0.088, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, a) and torch.equal(lse, la)  # o_lo changes nothing else
    o_ref, _ = oracle.attn_dense(q, k, v, scale=f32(0.088), causal=causal)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), scale=f32(0.088), causal=causal)
    check_o_lo("o_lo_%s_causal%d" % (dtype, causal), o, lo, o_ref, o_abs, q.dtype, 300)


@pytest.mark.parametrize("D", [64, 128])
def test_padded_query_blocks_with_o_lo(D):
    # A short batch leaves whole 256-row query blocks past its length: their
    # rows (padding up to Sq) get O = 0, LSE = -inf and o_lo = 0 without the
    # tile pipeline; the other rows match the oracle. Poisoned outputs show
    # any row that is not written.
    _, q, k, v = synth.dense_inputs(520 + D, 2, 4, 2, 700, 650, D, D, "bf16")
    sq = torch.tensor([700, 190], dtype=torch.int32)
    sk = torch.tensor([650, 120], dtype=torch.int32)
    qg, kg, vg, sqg, skg = gpu(q, k, v, sq, sk)
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full(q.shape[:3], 7.0, dtype=torch.float32, device="cuda")
    lo = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    for causal in (False, True):
        fa.fa_fwd(qg, kg, vg, scale=0.1, causal=causal, seqlens_q=sqg, seqlens_k=skg, out=o, lse=lse, o_lo=lo)
        torch.cuda.synchronize()
        assert torch.all(o[1, :, 190:] == 0) and torch.all(lo[1, :, 190:] == 0)
        assert torch.all(lse[1, :, 190:] == -math.inf)
        assert not torch.isnan(o).any() and not torch.isnan(lo).any()
        kw = dict(scale=f32(0.1), causal=causal, seqlens_q=sq, seqlens_k=sk)
        o_ref, lse_ref = oracle.attn_dense(q, k, v, **kw)
        o_abs, _ = oracle.attn_dense(q, k, absv(v), **kw)
        check("padded_blocks_D%d_causal%d" % (D, causal), o, lse, o_ref, lse_ref, q.dtype, o_abs)


def test_o_lo_full_causal_bf16_s4096():
    w = synth.workload("causal_bf16_s4096")
    q, k, v = w["q"], w["k"], w["v"]
    o, lse, lo = fa.fa_fwd(*gpu(q, k, v), scale=w["scale"], causal=True, return_o_lo=True)
    torch.cuda.synchronize()
    B, Hq, Sq, D = q.shape
    rows = sample_rows(np.random.default_rng(4321), B * Hq * Sq, 256, [0, Sq - 1])
    kw = dict(scale=f32(w["scale"]), causal=True, rows=rows)
    o_ref, _ = oracle.attn_dense(q, k, v, **kw)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), **kw)
    idx = torch.from_numpy(rows).cuda()
    check_o_lo("o_lo_full_causal_bf16_s4096", o.reshape(-1, D)[idx], lo.reshape(-1, D)[idx], o_ref, o_abs,
               q.dtype, Sq)
