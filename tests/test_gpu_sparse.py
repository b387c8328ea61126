"""GPU parity of fa_fwd_blocksparse and fa_fwd_topk_gather against the fp64
oracle, plus the order-invariance gates of the exact running max."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import check, f32, gpu, log, sample_rows
from oracle import metrics

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- block-sparse

def run_bs(case, q, k, v, lists, scale, seqlens=None):
    o, lse = fa.fa_fwd_blocksparse(*gpu(q, k, v), gpu(lists), scale=scale, seqlens=gpu(seqlens))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_blocksparse(q, k, v, lists, scale=f32(scale), seqlens=seqlens)
    o_abs, _ = oracle.attn_blocksparse(q, k, v.abs(), lists, scale=f32(scale), seqlens=seqlens)
    return check(case, o, lse, o_ref, lse_ref, q.dtype, o_abs)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_blocksparse_small(dtype, G):
    S = 700  # 6 query blocks, last one ragged
    g, q, k, v = synth.dense_inputs(30 + G, 2, 4 * G if G > 1 else 3, 4 if G > 1 else 3, S, S, 128,
                                    128, dtype)
    lists = synth.causal_block_lists(g, 6, 4)
    lists[2] = torch.tensor([-1, 0, -1, 2], dtype=torch.int32)  # holes anywhere
    lists[4] = torch.tensor([-1, -1, -1, -1], dtype=torch.int32)  # empty list -> zero rows
    seq = torch.tensor([S, 450], dtype=torch.int32)
    run_bs("bs_%s_G%d" % (dtype, G), q, k, v, lists, 1 / math.sqrt(128), seq)


def test_blocksparse_all_blocks_equals_dense():
    g, q, k, v = synth.dense_inputs(40, 1, 4, 2, 512, 512, 128, 128, "f16")
    lists = torch.stack([torch.randperm(4, generator=torch.Generator().manual_seed(i)) for i in range(4)]).int()
    rep = run_bs("bs_all_blocks", q, k, v, lists, 0.1)
    od, ld = fa.fa_fwd(*gpu(q, k, v), scale=0.1)
    os_, ls_ = fa.fa_fwd_blocksparse(*gpu(q, k, v), gpu(lists), scale=0.1)
    torch.cuda.synchronize()
    # same keys, different tile order: equal within the rounding of P
    assert metrics.rel_l2(os_.float().cpu(), od.float().cpu()) < 2e-3
    assert rep["rows"] == 4 * 512


def test_blocksparse_per_head_lists_d64():
    g, q, k, v = synth.dense_inputs(41, 2, 4, 2, 256, 384, 64, 64, "bf16")
    lists = torch.full((2, 2, 2, 3), -1, dtype=torch.int32)
    for b in range(2):
        for h in range(2):
            for qb in range(2):
                n = int(g.integers(1, 4))
                lists[b, h, qb, :n] = torch.from_numpy(g.choice(3, n, replace=False).astype(np.int32))
    run_bs("bs_per_head_d64", q, k, v, lists, 0.125)


def test_full_blocksparse_f16_s8192():
    # Exact running max (the contract path) and lazy rescale on the same
    # inputs; fp16 at full size: the literal atol/rtol gate on every sampled
    # element.
    w = synth.workload("blocksparse_f16_s8192")
    q, k, v = w["q"], w["k"], w["v"]
    qg, kg, vg, bi, sl = gpu(q, k, v, w["block_idx"], w["seqlens"])
    B, Hq, S, D = q.shape
    g = np.random.default_rng(77)
    must = [0, S - 1, S + 4999, S + 5000, 2 * S - 1, (2 * Hq - 1) * S + 4990]  # around seqlen 5000
    rows = sample_rows(g, B * Hq * S, 384, must)
    kw = dict(scale=f32(w["scale"]), seqlens=w["seqlens"], rows=rows)
    o_ref, lse_ref = oracle.attn_blocksparse(q, k, v, w["block_idx"], **kw)
    o_abs, _ = oracle.attn_blocksparse(q, k, v.abs(), w["block_idx"], **kw)
    idx = torch.from_numpy(rows).cuda()
    for thr in (0.0, 8.0):
        o, lse = fa.fa_fwd_blocksparse(qg, kg, vg, bi, scale=w["scale"], seqlens=sl, rescale_threshold=thr)
        torch.cuda.synchronize()
        check("full_blocksparse_f16_s8192_thr%g" % thr, o.reshape(-1, D)[idx], lse.reshape(-1)[idx], o_ref,
              lse_ref, torch.float16, o_abs, {"sampled_rows": len(rows), "rescale_threshold": thr}, plain_cap=0.0,
              page_gate=True)
        # padded rows of batch 1 (i >= 5000) are exactly zero / -inf everywhere
        assert torch.all(o[1, :, 5000:] == 0) and torch.all(torch.isneginf(lse[1, :, 5000:]))
        assert torch.all(torch.isfinite(lse[0])) and torch.all(torch.isfinite(lse[1, :, :5000]))
        assert not torch.isnan(o).any()


# ---------------------------------------------------------------- top-k MLA

def run_topk(case, q, kv, idx, scale, dv=512, alias=True, rows=None):
    qg, kg, ig = gpu(q, kv, idx)
    vg = kg[:, :dv] if alias else kg[:, :dv].contiguous()
    o, lse = fa.fa_fwd_topk_gather(qg, kg, vg, ig, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_topk(q, kv, kv[:, :dv], idx, scale=f32(scale), rows=rows)
    o_abs, _ = oracle.attn_topk(q, kv, kv[:, :dv].abs(), idx, scale=f32(scale), rows=rows)
    if rows is not None:
        r = torch.from_numpy(rows).cuda()
        o, lse = o.reshape(-1, dv)[r], lse.reshape(-1)[r]
    return o, lse, o_ref, lse_ref, o_abs


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("alias", [True, False])
def test_topk_small(dtype, alias):
    w = synth.topk_mla(50, 200, 300, 100, 64, 576, 512, dtype=dtype)
    idx = w["idx_a"].clone()
    idx[3, 5:20] = -1  # holes in the middle of a row
    idx[7] = -1        # a row with no key -> O = 0, LSE = -inf
    o, lse, o_ref, lse_ref, o_abs = run_topk("topk_small", w["q"], w["kv"], idx, w["scale"], alias=alias)
    check("topk_%s_alias%d" % (dtype, alias), o, lse, o_ref, lse_ref, w["q"].dtype, o_abs)


def test_topk_prefix_lists_equal_causal_dense():
    # idx[t] = 0..t is causal attention over one KV head (D = 576 / 512 split)
    w = synth.topk_mla(51, 96, 96, 96, 32, 576, 512)
    T = 96
    idx = torch.full((T, T), -1, dtype=torch.int32)
    for t in range(T):
        idx[t, :t + 1] = torch.arange(t + 1, dtype=torch.int32)
    o, lse, o_ref, lse_ref, o_abs = run_topk("topk_prefix", w["q"], w["kv"], idx, w["scale"])
    check("topk_prefix_causal", o, lse, o_ref, lse_ref, torch.bfloat16, o_abs)


def _order_gates(name, w, rows, rep_extra=None, plain_cap=None):
    """Both index orders against the oracle, row gain <= 2F each, and the
    coherent part of their difference <= 2F (exact running max)."""
    outs = {}
    for order in ("idx_a", "idx_b"):
        o, lse, o_ref, lse_ref, o_abs = run_topk(name, w["q"], w["kv"], w[order], w["scale"], rows=rows)
        rep = check("%s_%s" % (name, order), o, lse, o_ref, lse_ref, torch.bfloat16, o_abs, rep_extra,
                    plain_cap=plain_cap)
        outs[order] = o.float().cpu().numpy().astype(np.float64)
    F = metrics.bf16_floor(o_ref)
    ga = metrics.rms(metrics.row_gain(outs["idx_a"], o_ref))
    gb = metrics.rms(metrics.row_gain(outs["idx_b"], o_ref))
    gd = metrics.rms(metrics.row_gain(outs["idx_a"] - outs["idx_b"] + o_ref, o_ref))
    log(name + "_order_gates", {"floor_F": F, "gain_a_over_F": ga / F, "gain_b_over_F": gb / F,
                                "order_diff_over_F": gd / F})
    assert ga <= 2 * F and gb <= 2 * F and gd <= 2 * F


def test_topk_order_invariance_small():
    w = synth.topk_mla(52, 300, 300, 128, 64, 576, 512, peak_dims=576)
    _order_gates("topk_order_small", w, None)


def test_full_topk_mla_bf16_t4096():
    w = synth.workload("topk_mla_bf16_t4096")
    g = np.random.default_rng(5)
    T, Hq = w["q"].shape[:2]
    toks = np.sort(g.choice(T, size=24, replace=False))
    rows = (toks[:, None] * Hq + np.arange(Hq)[None, :]).reshape(-1)
    _order_gates("full_topk_mla_bf16_t4096", w, rows, {"sampled_tokens": len(toks)}, plain_cap=0.006)


@pytest.mark.parametrize("hq", [16, 40])
def test_topk_query_heads_not_a_multiple_of_32(hq):
    # Query heads padded to the wave's 32: the padding heads compute on a real
    # head and store nothing; heads past Hq are never written.
    w = synth.topk_mla(53, 64, 200, 96, hq, 576, 512)
    qg, kg, ig = gpu(w["q"], w["kv"], w["idx_a"])
    full = torch.full((64, hq + 8, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    o = full[:, :hq]
    lse = torch.empty((64, hq), dtype=torch.float32, device="cuda")
    fa.fa_fwd_topk_gather(qg, kg, kg[:, :512], ig, scale=w["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(full[:, hq:] == 7.0)
    o_ref, lse_ref = oracle.attn_topk(w["q"], w["kv"], w["kv"][:, :512], w["idx_a"], scale=f32(w["scale"]))
    o_abs, _ = oracle.attn_topk(w["q"], w["kv"], w["kv"][:, :512].abs(), w["idx_a"], scale=f32(w["scale"]))
    check("topk_hq%d" % hq, o, lse, o_ref, lse_ref, torch.bfloat16, o_abs)


def test_topk_o_lo():
    from test_gpu_dense import check_o_lo
    w = synth.topk_mla(54, 96, 300, 128, 64, 576, 512)
    qg, kg, ig = gpu(w["q"], w["kv"], w["idx_b"])
    o, lse, lo = fa.fa_fwd_topk_gather(qg, kg, kg[:, :512], ig, scale=w["scale"], return_o_lo=True)
    a, la = fa.fa_fwd_topk_gather(qg, kg, kg[:, :512], ig, scale=w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o, a) and torch.equal(lse, la)
    o_ref, _ = oracle.attn_topk(w["q"], w["kv"], w["kv"][:, :512], w["idx_b"], scale=f32(w["scale"]))
    o_abs, _ = oracle.attn_topk(w["q"], w["kv"], w["kv"][:, :512].abs(), w["idx_b"], scale=f32(w["scale"]))
    check_o_lo("topk_o_lo", o, lo, o_ref, o_abs, torch.bfloat16, 128)
