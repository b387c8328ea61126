"""The allocation-free split-KV entry point (fa_fwd_splitkv_noalloc) against
fa_fwd_splitkv with a caller workspace, through the C ABI: the same key ranges
give the same kernels on the same inputs, so the results must be identical
bit for bit, on two calls in a row (the second one smaller, reusing the
static scratch the first one left), and both meet the oracle's gates."""
import math

import numpy as np
import pytest
import torch

import flashattention_online_softmax_amd as fa
import oracle
import synth
from fa_testutil import check, f32, gpu

pytestmark = pytest.mark.gpu


def _pair(q, k, v, scale, causal, num_splits, sk=None):
    qg, kg, vg = gpu(q, k, v)
    skg = gpu(sk)
    B, Hq, Sq, D = q.shape
    a = torch.empty((B, Hq, Sq, D), dtype=q.dtype, device="cuda")
    la = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, 5.0)
    lb = torch.full_like(la, 5.0)
    fa.fa_fwd_splitkv(qg, kg, vg, scale=scale, causal=causal, seqlens_k=skg, num_splits=num_splits, out=a, lse=la)
    fa.fa_fwd_splitkv_noalloc(qg, kg, vg, scale=scale, causal=causal, seqlens_k=skg, num_splits=num_splits,
                              out=b, lse=lb)
    torch.cuda.synchronize()
    return a, la, b, lb


def test_noalloc_matches_workspace_entry_point_twice():
    # call 1: 4 ranges over 3000 keys, 2 x 8 heads x 300 rows
    _, q, k, v = synth.dense_inputs(700, 2, 8, 2, 300, 3000, 128, 128, "bf16")
    ns = fa.splitkv_splits(2, 8, 300, 3000, 4)
    assert ns == 4
    a, la, b, lb = _pair(q, k, v, 1 / math.sqrt(128), True, 4)
    assert torch.equal(a, b) and torch.equal(la, lb)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=f32(1 / math.sqrt(128)), causal=True)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), scale=f32(1 / math.sqrt(128)), causal=True)
    check("noalloc_call1", b, lb, o_ref, lse_ref, torch.bfloat16, o_abs)
    # call 2, smaller: fewer rows and keys, other lengths per batch, fp16, D = 64
    _, q, k, v = synth.dense_inputs(701, 2, 4, 4, 70, 1500, 64, 64, "f16")
    sk = torch.tensor([1500, 400], dtype=torch.int32)
    a, la, b, lb = _pair(q, k, v, 0.125, False, 3, sk)
    assert torch.equal(a, b) and torch.equal(la, lb)
    o_ref, lse_ref = oracle.attn_dense(q, k, v, scale=0.125, seqlens_k=sk)
    o_abs, _ = oracle.attn_dense(q, k, v.abs(), scale=0.125, seqlens_k=sk)
    check("noalloc_call2", b, lb, o_ref, lse_ref, torch.float16, o_abs)


def test_noalloc_rejects_problems_beyond_the_scratch():
    # 64 ranges x 2 x 32 x 1024 rows x 129 floats > 16M floats: refused, nothing written
    q = torch.zeros((2, 32, 1024, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 32, 64 * 192, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 2.0)
    lse = torch.full((2, 32, 1024), 2.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError, match="static scratch"):
        fa.fa_fwd_splitkv_noalloc(q, k, k, scale=0.1, num_splits=64, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 2.0) and torch.all(lse == 2.0)
