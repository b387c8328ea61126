// Work decomposition and tile bookkeeping shared by the attention forward
// kernels: workgroup-to-(batch, head, query block) mapping, the number of
// key tiles a query block visits (dense / causal / block-sparse), and the
// LDS chunk swizzles of K and V tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

constexpr int BN = 64;  // keys per block-sparse tile (half a 128-key block)

// 16-byte chunk swizzles (chunk index XOR f(row)) of the K and V tiles.
// K is read 16 bytes per lane by 32 lanes at 32 consecutive rows of one chunk
// column; V is read 8 bytes per lane by ds_read_b64_tr_b16 at 4 consecutive
// rows and 4 consecutive chunks per half wave.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Key held by LDS tile row `slot` in the key-permuted tile layout of the
// kernels with LDS-staged boolean masks. The S^T accumulator of a 32-key half
// gives lane (h, c) the rows 8 g + 4 h + i (g, i in 0..3); storing key
// 16 h + 4 g + i in row 8 g + 4 h + i hands that lane the 16 consecutive keys
// 16 h .. 16 h + 15, whose mask bytes are one 16-byte chunk. V tiles use the
// same rows, so P V pairs every p with its own key.
__device__ __forceinline__ int perm_key(int slot) {
  return (slot & ~31) | (((slot >> 2) & 1) << 4) | (((slot >> 3) & 3) << 2) | (slot & 3);
}

struct Work {
  int b, hkv, hq, wg_row0, row0, Lq, Lk;
  int qoff, koff;  // packed layout: first row of the batch in q / k (else 0)
  int split;       // split-KV: the key range index (else 0)
};

// Decodes blockIdx.x into (query block, head group, KV head, batch); the
// last query block comes first (longest causal rows first) and the KV-head
// index varies fastest, so the query heads of one KV head share an XCD
// (workgroup i runs on XCD i % 8), and the head groups of a KV head share
// its XCD and read its K/V tiles through one L2. Batches of different
// lengths (per-batch sequence lengths) run sequence-major (below).
//
// XM selects the extra modes of the 16-bit kernels: 1 = packed
// variable-length batches (row and key offsets and lengths from cu_q / cu_k;
// sequence-major order, below), 2 = split-KV (the split index varies slower
// than the head and faster than the query block, or pair-major, below; with
// per-batch lengths head group g takes the (batch, KV head) pairs rotated by
// g * B Hkv / n_hgroups, so that a short batch does not leave whole XCDs
// idle).
template <int NW, int QT, int HP, int XM = 0>
__device__ __forceinline__ Work decode_work(const FwdParams& p) {
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * QT * 32;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform: scalar
  const int BHkv = p.B * p.Hkv;
  const int per_mb = BHkv * p.n_hgroups;
  const int id = blockIdx.x;
  int mb_rank, r, split = 0;
  if (XM == 1 || (XM == 0 && (p.seqlens_q || p.seqlens_k))) {
    // Packed sequences, and batches of different lengths: sequence-major (all
    // query blocks and heads of one sequence before the next, longest blocks
    // first within it), so that each XCD works on one sequence's K/V at a
    // time instead of on blocks of many sequences whose K/V together
    // overflow its L2, and so that the workgroups that follow each other on
    // an XCD cost about the same. (Each XCD hands its workgroups to its
    // shader engines in turn and in order, waiting while the next engine in
    // turn is full: a pattern in which every other workgroup of an XCD is
    // short, as (batch, head group) pairs alternating between a long and a
    // short batch give, leaves half of the engines idle.)
    const int per_seq = p.n_mblocks * p.Hkv * p.n_hgroups;
    const int b = id / per_seq;
    const int r1 = id - b * per_seq;
    mb_rank = r1 / (p.Hkv * p.n_hgroups);
    r = b * p.Hkv + (r1 - mb_rank * (p.Hkv * p.n_hgroups)) % p.Hkv +
        ((r1 - mb_rank * (p.Hkv * p.n_hgroups)) / p.Hkv) * BHkv;
  } else if (XM == 2 && !(p.seqlens_q || p.seqlens_k) && BHkv % 8 == 0) {
    // Split-KV over equal-length batches: pair-major per XCD. Workgroup i
    // runs on XCD i % 8, which keeps the (batch, KV head) pair i % 8 (mod 8),
    // and the XCD works through its pairs one key range at a time (every
    // query block and head group of the range together), so the workgroups
    // reading one range's K/V run concurrently and share the XCD's L2. (The
    // plain kernels keep the query-block-major order: there the global
    // longest-first order balances causal work better than this locality
    // gains, 0.147 against 0.192 ms for causal S = 4096.)
    const int xcd = id & 7;
    int rest = id >> 3;
    const int ng = p.n_hgroups;
    const int hg0 = rest % ng;
    rest /= ng;
    mb_rank = rest % p.n_mblocks;
    rest /= p.n_mblocks;
    const int pair_hi = rest % (BHkv >> 3);
    if (XM == 2) split = rest / (BHkv >> 3);
    r = hg0 * BHkv + pair_hi * 8 + xcd;
  } else if (XM == 2) {
    const int per = per_mb * p.n_splits;
    mb_rank = id / per;
    const int r2 = id - mb_rank * per;
    split = r2 / per_mb;
    r = r2 - split * per_mb;
  } else {
    mb_rank = id / per_mb;
    r = id - mb_rank * per_mb;
  }
  const int mb = p.n_mblocks - 1 - mb_rank;
  const int hg = r / BHkv;
  const bool ragged = XM == 2 && (p.seqlens_q || p.seqlens_k);
  const int bkv = ragged ? (r - hg * BHkv + hg * (BHkv / p.n_hgroups)) % BHkv : r - hg * BHkv;
  Work wk;
  wk.b = bkv / p.Hkv;
  wk.hkv = bkv - wk.b * p.Hkv;
  const int hp = w / WPH, wi = w - (w / WPH) * WPH;
  wk.hq = wk.hkv * p.G + hg * HP + hp;
  wk.wg_row0 = mb * MPH;
  wk.row0 = wk.wg_row0 + wi * QT * 32;
  int lq = p.Sq, lk = p.Skv;
  wk.qoff = 0;
  wk.koff = 0;
  wk.split = split;
  if (XM == 1) {
    wk.qoff = p.cu_q[wk.b];
    wk.koff = p.cu_k[wk.b];
    lq = max(0, min(p.cu_q[wk.b + 1] - wk.qoff, p.Sq));
    lk = max(0, p.cu_k[wk.b + 1] - wk.koff);
  } else {
    if (p.seqlens_q) lq = max(0, min(p.seqlens_q[wk.b], p.Sq));
    if (p.seqlens_k) lk = max(0, min(p.seqlens_k[wk.b], p.Skv));
  }
  wk.Lq = lq;
  wk.Lk = lk;
  return wk;
}

// Block-sparse: compacts the valid entries of this query block's list into
// key-tile start offsets in LDS (first the first halves of every listed
// 128-key block, then the second halves that lie below Lk). Returns the
// number of 64-key tiles. Executed by wave 0; all waves read the result after
// the barrier.
__device__ __forceinline__ int build_sparse_tiles(const FwdParams& p, const Work& wk, int qb,
                                                  int* s_kstart, int* s_n) {
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    int n1 = 0, n2 = 0;
    const int32_t* list = p.block_idx + wk.b * p.bi_sb + wk.hkv * p.bi_sh + (int64_t)qb * p.bi_sq;
    // pass 1 counts first halves, pass 2 second halves
    for (int pass = 0; pass < 2; ++pass) {
      for (int s0 = 0; s0 < p.max_sel; s0 += 64) {
        const int s = s0 + lane;
        int x = -1;
        if (s < p.max_sel && wk.wg_row0 < wk.Lq) x = list[s];
        const int k0 = x * 128 + pass * 64;
        const bool ok = x >= 0 && k0 < wk.Lk;
        const uint64_t bal = __ballot(ok);
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        if (pass == 0) {
          if (ok) s_kstart[n1 + pos] = k0;
          n1 += __popcll(bal);
        } else {
          if (ok) s_kstart[n1 + n2 + pos] = k0;
          n2 += __popcll(bal);
        }
      }
    }
    if (lane == 0) *s_n = n1 + n2;
  }
  __syncthreads();
  return *s_n;
}

// Number of bn-key tiles of a dense (optionally causal) workgroup whose keys
// start at klo and end before wk.Lk; key j is visible to row i iff
// j <= i + diag under the causal mask.
template <bool CAUSAL>
__device__ __forceinline__ int dense_tiles(const Work& wk, int mph, int bn, int diag, int klo = 0) {
  if (wk.wg_row0 >= wk.Lq) return 0;
  int kend = wk.Lk;
  if (CAUSAL) {
    const int last_row = min(wk.wg_row0 + mph, wk.Lq) - 1;
    kend = min(kend, last_row + diag + 1);
  }
  return kend > klo ? (kend - klo + bn - 1) / bn : 0;
}

}  // namespace fa
