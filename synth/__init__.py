"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws inputs; it holds none of the attention arithmetic.
Every workload seed is split with numpy's SeedSequence into one child stream
per input in a fixed order (Q, K, V, then mask / row selection / block lists
/ indices); large tensors are drawn in fixed 4M-element chunks, each from its
own grandchild PCG64 stream, on a thread pool (the values depend only on the
seed and the shape, never on the thread count). Draws are float32 and are
rounded to the target dtype with round-to-nearest-even (torch ``.to``). The
same CPU tensors feed both the GPU library (after upload) and the oracle.

Named workloads (sizes as the pages' configurations give them):

  dense_f32_s128       fp32, B=1, H=1, S=128, D=64, no mask, scale 1/8
  causal_bf16_s4096    bf16 BNSD, B=2, H=16, S=4096, D=128, causal
  gqa_mask_f16_s8192   fp16 BNSD, B=4, Hq=32, Hkv=8, S=8192, D=128, causal
                       + Bernoulli(0.05) boolean mask (1 = masked, diagonal
                       kept) + 1% of query rows scaled x30
  blocksparse_f16_s8192 fp16, B=2, Hq=16, Hkv=4, S=8192, D=128, 128x128
                       blocks, 16 slots per query block (diagonal + up to 15
                       earlier blocks), seqlens [8192, 5000]
  topk_mla_bf16_t4096  bf16, T=S=4096, W=2048, Hq=128, Dqk=576 (512 latent +
                       64 rope), Dv=512, one shared KV head, V = K[:, :512],
                       self key + min(W-1, t) earlier keys per token
  causal_bf16_s8192    bf16 BNSD, B=2, H=16, S=8192, D=128, causal
  splitkv_bf16_q512_k65536  bf16 BNSD, B=1, Hq=32, Hkv=8, Sq=512, Skv=65536,
                       D=128, causal bottom-right (the last 512 rows of a
                       65536-token context: few query rows over many keys)
  varlen_bf16_b16      bf16 packed TND, 16 sequences with lengths drawn
                       uniformly from [64, 8192], Hq=32, Hkv=8, D=128, causal
"""
import concurrent.futures
import math
import os

import numpy as np
import torch

CHUNK = 1 << 22
_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


class Stream:
    """A seeded source of inputs: each call to ``child()`` hands out the next
    independent stream, in call order."""

    def __init__(self, seed):
        self._ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
        self._n = 0

    def child(self) -> np.random.SeedSequence:
        c = np.random.SeedSequence(self._ss.entropy, spawn_key=self._ss.spawn_key + (self._n,))
        self._n += 1
        return c

    def gen(self) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(self.child()))

    # numpy Generator API used by the helpers below, on a fresh child stream
    def choice(self, *a, **k):
        return self.gen().choice(*a, **k)

    def random(self, *a, **k):
        return self.gen().random(*a, **k)

    def integers(self, *a, **k):
        return self.gen().integers(*a, **k)


def rng(seed: int) -> Stream:
    return Stream(seed)


def normal(g: Stream, shape) -> np.ndarray:
    """float32 N(0, 1) draws of ``shape`` from the next child stream of ``g``."""
    ss = g.child()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = ss.spawn(nchunks)

    def fill(i):
        a, b = i * CHUNK, min(n, (i + 1) * CHUNK)
        np.random.Generator(np.random.PCG64(kids[i])).standard_normal(size=b - a, dtype=np.float32, out=out[a:b])

    list(_POOL.map(fill, range(nchunks)))
    return out.reshape(shape)


def cast(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def bernoulli_mask(g, Sq, Skv, density, keep_diagonal=True) -> torch.Tensor:
    """uint8 [Sq, Skv]; each entry is 1 (masked) with probability ``density``;
    mask[i, i] = 0 when ``keep_diagonal``."""
    m = np.empty((Sq, Skv), dtype=np.uint8)
    ss = g.child()
    step = max(1, CHUNK // max(Skv, 1))
    starts = list(range(0, Sq, step))
    kids = ss.spawn(len(starts))

    def fill(i):
        r0 = starts[i]
        r1 = min(Sq, r0 + step)
        gi = np.random.Generator(np.random.PCG64(kids[i]))
        m[r0:r1] = gi.random(size=(r1 - r0, Skv), dtype=np.float32) < density

    list(_POOL.map(fill, range(len(starts))))
    if keep_diagonal:
        d = np.arange(min(Sq, Skv))
        m[d, d] = 0
    return torch.from_numpy(m)


def pick_rows(g, nrows_total, frac) -> np.ndarray:
    """floor(frac * nrows_total) distinct flattened row ids, sorted."""
    n = int(math.floor(frac * nrows_total))
    return np.sort(g.gen().choice(nrows_total, size=n, replace=False)).astype(np.int64)


def causal_block_lists(g, nqb, max_sel) -> torch.Tensor:
    """int32 [nqb, max_sel]: query block i keeps KV block i plus min(max_sel-1, i)
    distinct earlier blocks drawn uniformly; ascending; unused slots -1."""
    out = np.full((nqb, max_sel), -1, dtype=np.int32)
    gg = g.gen()
    for i in range(nqb):
        extra = gg.choice(i, size=min(max_sel - 1, i), replace=False) if i > 0 else np.array([], np.int64)
        sel = np.sort(np.concatenate([extra, [i]]).astype(np.int32))
        out[i, :sel.size] = sel
    return torch.from_numpy(out)


def topk_indices(g, T, S, W):
    """Two int32 [T, W] index orders over the same key sets.

    Key set of token t: t itself plus min(W-1, t) distinct keys drawn uniformly
    from [0, t) (all of [0, t) when t < W).
      order A (self first): t, then the drawn keys ascending, then -1.
      order B (self last): the same keys fully ascending (t is the largest), then -1.
    """
    a = np.full((T, W), -1, dtype=np.int32)
    b = np.full((T, W), -1, dtype=np.int32)
    g = g.gen()
    for t in range(T):
        n = min(W - 1, t, S - 1) if S > 0 else 0
        if n == t:
            extra = np.arange(t, dtype=np.int32)
        else:
            extra = np.sort(g.choice(t, size=n, replace=False)).astype(np.int32)
        if t < S:
            a[t, 0] = t
            a[t, 1:1 + n] = extra
            b[t, :n] = extra
            b[t, n] = t
    return torch.from_numpy(a), torch.from_numpy(b)


def dense_inputs(seed, B, Hq, Hkv, Sq, Skv, D, Dv, dtype):
    g = rng(seed)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    q = cast(normal(g, (B, Hq, Sq, D)), dt)
    k = cast(normal(g, (B, Hkv, Skv, D)), dt)
    v = cast(normal(g, (B, Hkv, Skv, Dv)), dt)
    return g, q, k, v


def workload(name: str) -> dict:
    """Full-size named workload as a dict of CPU tensors and parameters."""
    if name == "dense_f32_s128":
        g, q, k, v = dense_inputs(1, 1, 1, 1, 128, 128, 64, 64, "f32")
        return dict(kind="dense", q=q, k=k, v=v, scale=1.0 / math.sqrt(64), causal=False)
    if name == "causal_bf16_s4096":
        g, q, k, v = dense_inputs(2, 2, 16, 16, 4096, 4096, 128, 128, "bf16")
        return dict(kind="dense", q=q, k=k, v=v, scale=1.0 / math.sqrt(128), causal=True)
    if name == "causal_bf16_s8192":
        g, q, k, v = dense_inputs(6, 2, 16, 16, 8192, 8192, 128, 128, "bf16")
        return dict(kind="dense", q=q, k=k, v=v, scale=1.0 / math.sqrt(128), causal=True)
    if name == "gqa_mask_f16_s8192":
        return gqa_mask(3, 4, 32, 8, 8192, 128)
    if name == "blocksparse_f16_s8192":
        return blocksparse(4, 2, 16, 4, 8192, 128, [8192, 5000])
    if name == "topk_mla_bf16_t4096":
        return topk_mla(5, 4096, 4096, 2048, 128, 576, 512)
    if name == "splitkv_bf16_q512_k65536":
        g, q, k, v = dense_inputs(7, 1, 32, 8, 512, 65536, 128, 128, "bf16")
        return dict(kind="dense", q=q, k=k, v=v, scale=1.0 / math.sqrt(128), causal=True, split=True)
    if name == "varlen_bf16_b16":
        return varlen(8, 16, 64, 8192, 32, 8, 128)
    raise KeyError(name)


def varlen(seed, B, lmin, lmax, Hq, Hkv, D, dtype="bf16", causal=True, lens_q=None, lens_k=None):
    """Packed (TND) variable-length batch: sequence lengths drawn uniformly
    from [lmin, lmax] unless lens_q is given (self-attention: keys of the same
    lengths unless lens_k is given); q [Tq, Hq, D], k/v [Tk, Hkv, D],
    cu_seqlens int32 [B+1]."""
    g = rng(seed)
    lens = g.integers(lmin, lmax + 1, size=B).astype(np.int64)
    if lens_q is not None:
        lens = np.asarray(lens_q, dtype=np.int64)
    lk = lens if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    dt = DTYPES[dtype]
    Tq, Tk = int(lens.sum()), int(lk.sum())
    q = cast(normal(g, (Tq, Hq, D)), dt)
    k = cast(normal(g, (Tk, Hkv, D)), dt)
    v = cast(normal(g, (Tk, Hkv, D)), dt)
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(lk)]).astype(np.int32))
    return dict(kind="varlen", q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, max_q=int(lens.max()),
                scale=1.0 / math.sqrt(D), causal=causal)


def gqa_mask(seed, B, Hq, Hkv, S, D, density=0.05, frac=0.01, factor=30.0, dtype="f16"):
    """GQA + causal + Bernoulli mask + a fraction of query rows scaled by ``factor``."""
    g = rng(seed)
    dt = DTYPES[dtype]
    q32 = normal(g, (B, Hq, S, D))
    k = cast(normal(g, (B, Hkv, S, D)), dt)
    v = cast(normal(g, (B, Hkv, S, D)), dt)
    mask = bernoulli_mask(g, S, S, density)
    rows = pick_rows(g, B * Hq * S, frac)
    q32.reshape(-1, D)[rows] *= np.float32(factor)
    q = cast(q32, dt)
    del q32
    return dict(kind="dense", q=q, k=k, v=v, scale=1.0 / math.sqrt(D), causal=True, mask=mask,
                scaled_rows=torch.from_numpy(rows))


def blocksparse(seed, B, Hq, Hkv, S, D, seqlens, block=128, max_sel=16, dtype="f16"):
    g, q, k, v = dense_inputs(seed, B, Hq, Hkv, S, S, D, D, dtype)
    nqb = (S + block - 1) // block
    lists = causal_block_lists(g, nqb, max_sel)
    return dict(kind="blocksparse", q=q, k=k, v=v, scale=1.0 / math.sqrt(D), block_idx=lists,
                block=block, seqlens=torch.tensor(seqlens, dtype=torch.int32))


def topk_mla(seed, T, S, W, Hq, Dqk, Dv, peak=0.25, peak_dims=None, dtype="bf16"):
    """Top-k sparse MLA inputs. q_t += peak * k_t on the first ``peak_dims``
    dims (default: the Dv latent dims) of every head."""
    g = rng(seed)
    dt = DTYPES[dtype]
    q32 = normal(g, (T, Hq, Dqk))
    k32 = normal(g, (S, Dqk))
    pd = Dv if peak_dims is None else peak_dims
    n = min(T, S)
    q32[:n, :, :pd] += np.float32(peak) * k32[:n, None, :pd]
    q = cast(q32, dt)
    k = cast(k32, dt)
    idx_a, idx_b = topk_indices(g, T, S, W)
    return dict(kind="topk", q=q, kv=k, dv=Dv, scale=1.0 / math.sqrt(Dqk), idx_a=idx_a,
                idx_b=idx_b)
