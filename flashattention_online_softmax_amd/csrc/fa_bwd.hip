// Attention backward for 16-bit inputs on gfx950 (D = 64 or 128; dense,
// causal, GQA): dQ, dK, dV from Q, K, V, the forward's O and LSE, and dO.
//
// Method: the backward formulas of the ops-transformer FlashAttentionScoreGrad
// pytest page (section 5.2) with the recomputation strategy of the PyPTO BSA
// README (section 3: the backward keeps only O and LSE and recomputes
// P = exp(scale S - LSE)):
//   P = exp2(scale log2e S - log2e LSE),  dP = dO V^T,  Delta_i = dO_i . O_i,
//   dS = P (dP - Delta),  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
// with dK and dV summed over the query heads of a KV head (BSA README,
// section 1).
//
// Packed variable-length batches (PK): each batch's rows and keys are a range
// of the packed [T, H, D] tensors given by cu_seqlens (the TND layout of the
// FlashAttentionScoreGrad pytest page, section 5.4); LSE and Delta are
// [Tq, Hq]. Rows and keys outside a batch's ranges are neither read as data
// nor written.
//
// No atomics. Without a dS workspace two kernels, dQ first (it also forms
// and stores Delta_i = dO_i . O_i in fp32, which the dK/dV kernel reads);
// with one, three: Delta (and the dK/dV kernel's per-tile start values),
// dK/dV storing dS, then dQ = scale dS K from the stored dS (bwd_dqg):
//   * dkdv: a workgroup owns 128 keys of one KV head (8 waves: for each 32
//     keys one wave computes S and P and accumulates dV, with K of its keys
//     resident as MFMA B operands, and one computes dP and dS and
//     accumulates dK, with V resident) and sweeps the query tiles (32 rows)
//     of every query head of the group: S = Q K^T, dP = dO V^T, then
//     dV^T += dO^T P and dK^T += Q^T dS on v_mfma_f32_32x32x16, P and dS
//     rounded to 16 bits as B operands straight from the accumulator layout.
//   * dq: a workgroup of 8 waves owns 256 query rows of one head (Q and dO
//     resident) and sweeps the key tiles: S^T = K Q^T, dP^T = V dO^T,
//     dQ^T += K^T dS^T.
// The operands read transposed (dO^T, Q^T, K^T) come from row-major LDS tiles
// through ds_read_b64_tr_b16, in the key (query) order in which the
// accumulator holds P and dS, so the contraction pairs the right elements.
// Each LDS tile is 32 rows x D, stored once with its 16-byte chunks
// XOR-swizzled so that both the row reads and the transposing reads are free
// of bank conflicts (bsw below).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_asm.h"
#include "fa_device.h"
#include "fa_bwd_params.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int TR = 32;     // rows of an LDS tile
constexpr int NWB = 4;     // 32-key groups per dK/dV workgroup (two waves each)
constexpr int BLK = 32 * NWB;  // keys per dK/dV workgroup
constexpr int NWQ = 8;         // waves per dQ workgroup (two per SIMD)
constexpr int BLKQ = 32 * NWQ;  // query rows per dQ workgroup

// One chunk swizzle serves both read patterns of a tile (256 bytes of LDS
// banks, 16 chunk positions).
// D = 128 (one row per 256 bytes): the row reads (16 consecutive rows, one
// chunk each) see 16 distinct chunk positions since the XOR term is a
// bijection of row & 15, and the transposing reads (4 consecutive rows x 4
// consecutive chunks) see 16 distinct positions since bits 2..3 of the XOR
// term differ between the four rows of an aligned group.
// D = 64 (two rows per 256 bytes, row parity picks the half): among 16
// consecutive rows the 8 of one parity get distinct XOR terms (a bijection
// of (row >> 1) & 7), so the row reads see 16 distinct positions; in an
// aligned group of 4 rows the two rows of one parity differ in bit 2 of the
// XOR term, so their 4 consecutive chunks land in opposite halves of the
// row and the transposing reads see 16 distinct positions too.
template <int BD>
__device__ __forceinline__ int bsw(int row, int ch) {
  if constexpr (BD == 128) return ch ^ (((row & 3) << 2) | ((row >> 2) & 3));
  return ch ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// A operand "rows": lane (c, h) holds tile row c, columns 16 ks + 8 h .. +7.
template <int BD>
__device__ __forceinline__ u32x4 row_op(const uint16_t* t, int ks) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  return *(const u32x4*)(t + c * BD + bsw<BD>(c, 2 * ks + h) * 8);
}
// A operand "transposed": M index = tile column 32 dt + (lane & 31); the 8 k
// values of lane half h are tile rows 16 ks + 4 h + 0..3 and 16 ks + 8 + 4 h
// + 0..3, the order in which a 32x32 accumulator holds its rows.
template <int BD>
__device__ __forceinline__ u32x4 tr_op(const uint16_t* t, int dt, int ks) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int vrow = 4 * h + ((lane & 15) >> 2);
  const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int r0 = 16 * ks + vrow, r1 = r0 + 8;
  const u32x2 lo = lds_read_tr16(t + r0 * BD + bsw<BD>(r0, col >> 3) * 8 + (col & 7));
  const u32x2 hi = lds_read_tr16(t + r1 * BD + bsw<BD>(r1, col >> 3) * 8 + (col & 7));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// B operand from global memory: lane (c, h) holds row r of a row-major
// matrix, columns 16 ks + 8 h .. +7, for the D / 16 k-steps over the head dim.
template <int BD>
__device__ __forceinline__ void load_bop(u32x4 (&op)[BD / 16], const uint16_t* base, int64_t stride, int r) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < BD / 16; ++ks) op[ks] = *(const u32x4*)(base + (int64_t)r * stride + 16 * ks + 8 * h);
}
// Accumulator elements 8 ks .. 8 ks + 7 rounded to 16 bits: the B operand of
// k-step ks over the accumulator's rows.
template <class T>
__device__ __forceinline__ u32x4 pack_b(const f32x16& a, int ks) {
  return u32x4{T::pack2(a[8 * ks], a[8 * ks + 1]), T::pack2(a[8 * ks + 2], a[8 * ks + 3]),
               T::pack2(a[8 * ks + 4], a[8 * ks + 5]), T::pack2(a[8 * ks + 6], a[8 * ks + 7])};
}
// Stores accumulator tiles acc[dt] (rows = head dim 32 dt + ..., column =
// lane's row r of the output) times mul as 16-bit values: 4 consecutive
// elements per store.
template <class T, int BD>
__device__ __forceinline__ void store_t(uint16_t* base, int64_t stride, int r, const f32x16 (&acc)[BD / 32], float mul) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int dt = 0; dt < BD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 v = {T::pack2(acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul),
                       T::pack2(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul)};
      *(u32x2*)(base + (int64_t)r * stride + 32 * dt + 8 * g + 4 * h) = v;
    }
}

// Sequence lengths of batch b (without the vectors: Sq and Skv).
__device__ __forceinline__ void batch_lengths(const BwdParams& p, int b, int& lq, int& lk) {
  lq = p.seqlens_q ? max(0, min(p.seqlens_q[b], p.Sq)) : p.Sq;
  lk = p.seqlens_k ? max(0, min(p.seqlens_k[b], p.Skv)) : p.Skv;
}

// Batch b's lengths and its first query row and key in the tensors: 0 and
// batch_lengths for the padded layout; from cu_seqlens for packed batches,
// clamped to the tensors' rows (so that offsets past them never address
// memory) and to the longest lengths the grid covers.
template <bool PK>
__device__ __forceinline__ void batch_geometry(const BwdParams& p, int b, int& lq, int& lk, int& qoff, int& koff) {
  if constexpr (PK) {
    qoff = min(max(p.cu_q[b], 0), p.Tq);
    koff = min(max(p.cu_k[b], 0), p.Tk);
    lq = max(0, min(min(p.cu_q[b + 1], p.Tq) - qoff, p.Sq));
    lk = max(0, min(min(p.cu_k[b + 1], p.Tk) - koff, p.Skv));
  } else {
    qoff = 0;
    koff = 0;
    batch_lengths(p, b, lq, lk);
  }
}
// Index of row i of query head hq of batch b in LSE and Delta: [B, Hq, Sq]
// (padded) or [Tq, Hq] (packed, qoff = the batch's first row).
template <bool PK>
__device__ __forceinline__ int64_t ld_index(const BwdParams& p, int b, int hq, int qoff, int i) {
  return PK ? (int64_t)(qoff + i) * p.Hq + hq : ((int64_t)b * p.Hq + hq) * p.Sq + i;
}

// End of a phase of the dK/dV kernel: the workgroup barrier, with no
// instruction of the phase (MFMAs included, which touch no memory) moved
// past it and none of the next phase moved before it.
__device__ __forceinline__ void phase_end() {
  __builtin_amdgcn_sched_barrier(0);
  barrier_keep_copies();
  __builtin_amdgcn_sched_barrier(0);
}

// Two waves per key group g of 32 keys (g = w % 4; waves g and g + 4 share
// a SIMD). The P wave (w < 4) holds K of its keys as B operands and dV^T;
// the dS wave (w >= 4) holds V and dK^T. Per step s of the sweep (a query
// head and a 32-row query tile):
//   M_P(s): S(s) = Q(s) K^T, and dV^T += dO(s-1)^T P(s-1)     (P wave)
//   V_P(s): P(s) = exp2(S scale log2e - LSE log2e), masked; stored in fp32
//           to LDS for the dS wave and rounded to 16 bits as the P wave's
//           next B operand
//   M_D(s): dP(s) = dO(s) V^T, and dK^T += Q(s-1)^T dS(s-1)    (dS wave)
//   V_D(s): dS(s) = P(s) (dP(s) - Delta), rounded to 16 bits
// The two waves run one phase apart and every phase ends with a workgroup
// barrier: phase 2s is M_P(s) with V_D(s-1), phase 2s+1 is V_P(s) with
// M_D(s). Every score is computed and exponentiated once and both waves
// issue 16 MFMAs per step. The transposed A operands of an M phase's
// gradient update (the slower transposing LDS reads, 8 KB per wave) are
// read during the wave's V phase before it, so on each SIMD they overlap
// the other wave's MFMAs; the row operands (Q or dO rows) are read at the
// start of the M phase, behind the update's MFMAs, which need no LDS.
//
// Tile lifetimes: Q(s) rows are read in phase 2s and dO(s) rows in phase
// 2s + 1; dO(s)^T in phase 2s + 1 (for M_P(s + 1)) and Q(s)^T in phase
// 2s + 2 (for M_D(s + 1)). The tiles live in a four-deep
// LDS ring (slot s % 4), copied HBM -> LDS by LDS-DMA (no register staging)
// by the P waves: at the start of phase 2t + 1 P wave g issues half a tile
// of step t + 3 (tile g / 2, chunk positions 64 (NPW (g % 2) + n) + lane,
// n < NPW = D / 32; the swizzle is an involution, so a lane fetches the
// logical chunk its position holds) into the slot of step t - 1, read last
// in phase 2t, and at the end of phase 2t it waits for its copies of step
// t + 1. S and dP start from -LSE / scale and -Delta of their rows (so V_P
// is one multiply and one exp2 per score and V_D one multiply per element,
// with no LDS read before them); these values of step s + 2 are loaded by
// wave 4 into registers during step s, stored into their ring slot at its
// end, and read at the start of the M phases of step s + 2.
template <class T, int BD, bool CAUSAL, bool MASK, bool PK, bool DSW>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NB = 4;  // ring depth
  constexpr int DT = BD / 32;   // 32-wide d tiles
  constexpr int CPR = BD / 8;   // 16-byte chunks per tile row
  constexpr int NPW = BD / 32;  // copy instructions per P wave and step (half a tile)
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[NB][2][TR * BD];
  __shared__ __attribute__((aligned(16))) float sLD[NB][2 * TR];  // -LSE / scale, then -Delta
  __shared__ __attribute__((aligned(16))) float pex[4][4][64][4];  // P of each key group
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 31, h = lane >> 5, g = w & 3;
  // (The wave index and everything selected by it are wave-uniform scalars,
  // so that the selects between kernel arguments stay in scalar registers.)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool dswave = wu >= 4;
  // Workgroups in order of decreasing work (under the causal mask the first
  // key blocks see the most query rows), the (batch, KV head) index fastest
  // so that one head's workgroups share an XCD (workgroup i runs on XCD i % 8).
  const int lin = blockIdx.x + blockIdx.y * gridDim.x, nbk = p.B * p.Hkv;
  const int bk = lin % nbk, b = bk / p.Hkv, hkv = bk % p.Hkv;
  const int k0 = (lin / nbk) * BLK;
  const int key = k0 + 32 * g + c;  // this lane's key (column of S)
  int Lq, Lk, qoff, koff;
  batch_geometry<PK>(p, b, Lq, Lk, qoff, koff);
  // A packed batch's key block past its keys has nothing to compute or write
  // (the rows there belong to the next batch).
  if (PK && k0 >= Lk) return;
  // Keys the lanes load and store: the padded tensors' rows, or the batch's.
  const int klim = PK ? Lk : p.Skv;
  const int diag = Lk - Lq;  // key j is visible to row i iff j <= i + diag
  const uint16_t* kg = (const uint16_t*)p.k + (int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh + (int64_t)koff * p.k_ss;
  const uint16_t* vg = (const uint16_t*)p.v + (int64_t)b * p.v_sb + (int64_t)hkv * p.v_sh + (int64_t)koff * p.v_ss;
  u32x4 kv_op[BD / 16];  // K (P wave) or V (dS wave) rows of the lane's key
  load_bop<BD>(kv_op, dswave ? vg : kg, dswave ? p.v_ss : p.k_ss, min(key, klim - 1));
  f32x16 acc[DT];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  // Query rows that can see a key of this block: i >= k0 - diag (causal),
  // swept from the multiple of 32 at or below, so that every 32 x 32 block
  // of dS that holds a visible element is stored whole (with the dS store)
  // and both dQ paths accumulate dK and dV in the same order.
  const int qfirst = CAUSAL ? max(0, k0 - diag) & ~(TR - 1) : 0;
  const int nqt = (k0 < Lk && Lq > qfirst) ? (Lq - qfirst + TR - 1) / TR : 0;
  // The sweep: step s = (query head hkv G + s / nqt, tile s % nqt).
  const int nsteps = p.G * nqt;
  // (h, t) of the step computed and of the step whose copies or LSE / Delta
  // come next, tracked without divisions.
  int h_cur = 0, t_cur = 0, h_ahd = 0, t_ahd = 0;
  auto advance = [&](int& hh, int& tt) __attribute__((always_inline)) {
    if (++tt == nqt) {
      tt = 0;
      ++hh;
    }
  };
  // P wave copies: tile (w & 3) / 2 (0 Q, 1 dO); per instruction the tile
  // row and the byte offset of the logical chunk.
  const bool c_do = (wu & 2) != 0;
  int crow[NPW];
  uint32_t cchunk[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    const int pos = 64 * (NPW * (wu & 1) + n) + lane, row = pos / CPR;
    crow[n] = row;
    cchunk[n] = (uint32_t)(bsw<BD>(row, pos % CPR) * 16);
  }
  const int64_t c_ss = c_do ? p.do_ss : p.q_ss, c_sh = c_do ? p.do_sh : p.q_sh;
  // the group's first query head
  const uint16_t* c_head =
      c_do ? (const uint16_t*)p.dout + (int64_t)b * p.do_sb + (int64_t)hkv * p.G * p.do_sh + (int64_t)qoff * p.do_ss
           : (const uint16_t*)p.q + (int64_t)b * p.q_sb + (int64_t)hkv * p.G * p.q_sh + (int64_t)qoff * p.q_ss;
  const int rlim = PK ? Lq : p.Sq;  // query rows the copies may read
  const uint32_t c_rb = (uint32_t)c_ss * 2u;
  const uint32_t c_lds = lds_addr_of(sbuf[0][c_do ? 1 : 0]) + (wu & 1) * (NPW * 1024);
  auto dma = [&](int hh, int tt, int sl) __attribute__((always_inline)) {
    const int q0 = qfirst + tt * TR;
    const uint16_t* base = c_head + (int64_t)hh * c_sh + (int64_t)q0 * c_ss;
    const int rmax = rlim - 1 - q0;  // rows past the last one fetch the last one
    const uint32_t l0 = c_lds + (uint32_t)sl * (2 * TR * BD * 2);
#pragma unroll
    for (int n = 0; n < NPW; ++n) lds_copy16(base, (uint32_t)min(crow[n], rmax) * c_rb + cchunk[n], l0 + n * 1024);
    // With the dS store, wave 0 also copies the step's 256-byte record of S
    // and dP start values (16 lanes of 16 bytes) into the LSE / Delta ring.
    if (DSW && wu == 0 && lane < 16)
      lds_copy16(p.ldrec + ((int64_t)(b * p.Hq + hkv * p.G + hh) * (p.ds_qp / TR) + q0 / TR) * (2 * TR),
                 (uint32_t)lane * 16u, lds_addr_of(sLD[sl]));
  };
  // Waits until this wave's copies of all but the last k issued steps are
  // complete (wave 0 issues one more copy per step with the dS store).
  auto wait_copies_below = [&](auto k) __attribute__((always_inline)) {
    if (DSW && wu == 0)
      wait_vmem_below<decltype(k)::value * (NPW + 1)>();
    else
      wait_vmem_below<decltype(k)::value * NPW>();
  };
  // Wave 4: lane i < 32 loads LSE of row q0 + i, lane 32 + i Delta; the
  // stored values (-LSE / scale and -Delta, the initial values of the S and
  // dP accumulators) are formed only when they are stored, so that the
  // load's latency hides behind the step.
  float ld = 0.f;
  const float inv_scale = -1.f / p.scale;
  auto fetch_ld = [&](int hh, int tt) __attribute__((always_inline)) {
    const int hq = hkv * p.G + hh, i = qfirst + tt * TR + c;
    const int64_t ri = ld_index<PK>(p, b, hq, qoff, i);
    ld = i >= rlim ? (h == 0 ? -INFINITY : 0.f) : h == 0 ? p.lse[ri] : p.delta[ri];
  };
  auto put_ld = [&](int sl) __attribute__((always_inline)) {
    // rows without keys (LSE = -inf) and padding rows get P = 0 (their
    // elements are masked; the +inf start keeps them out of any overflow)
    sLD[sl][lane] = h != 0 ? -ld : ld == -INFINITY ? INFINITY : ld * inv_scale;
  };
  // A operands of an M phase: the rows of one tile and the transposed other.
  u32x4 ar[BD / 16], at[BD / 16];
  auto read_rows = [&](const uint16_t* t) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < BD / 16; ++ks) ar[ks] = row_op<BD>(t, ks);
  };
  auto read_tr = [&](const uint16_t* t) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < BD / 16; ++ks) at[ks] = tr_op<BD>(t, ks % DT, ks / DT);
  };
  if (nsteps > 0) {
    if (!dswave) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < nsteps) {
          dma(h_ahd, t_ahd, j);
          advance(h_ahd, t_ahd);
        }
      // h_ahd, t_ahd: step 3; the copies of step 0 are complete
      if (nsteps > 2)
        wait_copies_below(std::integral_constant<int, 2>{});
      else if (nsteps > 1)
        wait_copies_below(std::integral_constant<int, 1>{});
      else
        wait_vmem();
    } else {
      if (!DSW && w == 4) {
        fetch_ld(0, 0);
        put_ld(0);
        if (nsteps > 1) {
          fetch_ld(0 + (nqt == 1), nqt == 1 ? 0 : 1);
          put_ld(1);
        }
      }
      advance(h_ahd, t_ahd);
      advance(h_ahd, t_ahd);  // step 2
    }
    barrier_keep_copies();
  }
  using F = std::false_type;
  using U = std::true_type;
  if (!dswave) {
    u32x4 pb[2];  // P(s - 1) as the B operand of the dV update
    f32x16 sv;
    // Phase 2s: M_P(s); phase 2s + 1: V_P(s) and the reads for M_P(s + 1).
    // DS: s < nsteps; DU: s > 0.
    auto step = [&](int s, auto DS, auto DU) __attribute__((always_inline)) {
      // S starts from -LSE / scale of its row, so that the exponent of P is
      // S scale log2e as it leaves the MFMAs.
      if (DS) {
        const float* sL = sLD[s & (NB - 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 l4 = *(const float4*)(sL + 8 * j + 4 * h);
          sv[4 * j] = l4.x; sv[4 * j + 1] = l4.y; sv[4 * j + 2] = l4.z; sv[4 * j + 3] = l4.w;
        }
        read_rows(sbuf[s & (NB - 1)][0]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (DU) {
#pragma unroll
        for (int ks = 0; ks < BD / 16; ++ks) acc[ks % DT] = T::mfma(at[ks], pb[ks / DT], acc[ks % DT]);
      }
      if (DS) {
#pragma unroll
        for (int ks = 0; ks < BD / 16; ++ks) sv = T::mfma(ar[ks], kv_op[ks], sv);
      }
      // This wave's copies of step s + 1 are complete (those of step s + 2
      // may still fly).
      if (s + 2 < nsteps)
        wait_copies_below(std::integral_constant<int, 1>{});
      else
        wait_vmem();
      phase_end();
      if (s + 3 < nsteps) dma(h_ahd, t_ahd, (s + 3) & (NB - 1));
      if (DS) {
        const int q0 = qfirst + t_cur * TR;
        read_tr(sbuf[s & (NB - 1)][1]);
        // Element i: query row q0 + r, r = 8 (i / 4) + 4 h + i % 4; key `key`.
        // A block every row and key of which exist and (causal) whose last
        // key the first row sees needs no per-element test.
        const int kw0 = k0 + 32 * g;
        const bool inside = !MASK && __builtin_amdgcn_readfirstlane(
                                         (kw0 + 31 < Lk && q0 + TR <= Lq && (!CAUSAL || kw0 + 31 <= q0 + diag)) ? 1 : 0);
        f32x16 pv;
        if (inside) {
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(sv[i] * p.scale_log2);
        } else {
          const uint8_t* mk = MASK ? p.mask + (int64_t)b * p.m_sb + (int64_t)(hkv * p.G + h_cur) * p.m_sh + key : nullptr;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = q0 + 8 * (i >> 2) + 4 * h + (i & 3);
            bool ok = key < Lk && qi < Lq;
            if (CAUSAL) ok = ok && key <= qi + diag;
            if (MASK) ok = ok && mk[(int64_t)qi * p.m_ss] == 0;
            pv[i] = ok ? fast_exp2(sv[i] * p.scale_log2) : 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(float4*)pex[g][j][lane] = make_float4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
        pb[0] = pack_b<T>(pv, 0);
        pb[1] = pack_b<T>(pv, 1);
      }
      phase_end();
      advance(h_cur, t_cur);
      advance(h_ahd, t_ahd);
    };
    if (nsteps > 0) {
      step(0, U{}, F{});
      for (int s = 1; s < nsteps; ++s) step(s, U{}, U{});
      step(nsteps, F{}, U{});
    }
  } else {
    u32x4 db[2];  // dS(s - 1) as the B operand of the dK update
    f32x16 dp;
    // (query head, tile) of the step whose dS is formed; only 32-key groups
    // that hold keys of the batch are stored (the dQ product reads no other).
    int h_ds = 0, t_ds = 0;
    const bool ds_store = DSW && k0 + 32 * g < Lk;
    const bool ds_nt = __builtin_amdgcn_readfirstlane(p.ds_nt) != 0;
    // Phase 2s: V_D(s - 1) and the reads for M_D(s); phase 2s + 1: M_D(s).
    // DS: s < nsteps; DU: s > 0.
    auto step = [&](int s, auto DS, auto DU) __attribute__((always_inline)) {
      const bool ldw = !DSW && w == 4 && s + 2 < nsteps;
      if (ldw) fetch_ld(h_ahd, t_ahd);
      if (DU) {
        float4 p4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p4[j] = *(const float4*)pex[g][j][lane];
        read_tr(sbuf[(s - 1) & (NB - 1)][0]);
        f32x16 dsv;  // dp holds dP - Delta
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dsv[4 * j] = p4[j].x * dp[4 * j];
          dsv[4 * j + 1] = p4[j].y * dp[4 * j + 1];
          dsv[4 * j + 2] = p4[j].z * dp[4 * j + 2];
          dsv[4 * j + 3] = p4[j].w * dp[4 * j + 3];
        }
        db[0] = pack_b<T>(dsv, 0);
        db[1] = pack_b<T>(dsv, 1);
        if (ds_store) {
          // The step's 32 x 32 block of dS: one contiguous 2 KB block, 64
          // bytes per key, the lane's 16 rows (accumulator order: element i
          // is row 8 (i / 4) + 4 h + i % 4) at positions 16 h + i, so each
          // lane stores 32 contiguous bytes. Non-temporal when the stored dS
          // outgrows the last-level cache: then it must not evict this
          // kernel's tiles from the L2 on its way to memory; below that the
          // dQ kernel finds it in the cache.
          const int q0s = qfirst + t_ds * TR;
          const int64_t blk = (((int64_t)(b * p.Hq + hkv * p.G + h_ds) * p.ds_nrb + (q0s >> 8)) * p.ds_nkt +
                               (k0 >> 5) + g) * 8 + ((q0s >> 5) & 7);
          u32x4* dst = (u32x4*)(p.ds + blk * 1024 + c * 32 + 16 * h);
          if (ds_nt) {
            __builtin_nontemporal_store(db[0], dst);
            __builtin_nontemporal_store(db[1], dst + 1);
          } else {
            dst[0] = db[0];
            dst[1] = db[1];
          }
        }
        advance(h_ds, t_ds);
      }
      phase_end();
      // dP starts from -Delta of its row.
      if (DS) {
        const float* sD = sLD[s & (NB - 1)] + TR;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 d4 = *(const float4*)(sD + 8 * j + 4 * h);
          dp[4 * j] = d4.x; dp[4 * j + 1] = d4.y; dp[4 * j + 2] = d4.z; dp[4 * j + 3] = d4.w;
        }
        read_rows(sbuf[s & (NB - 1)][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (DU) {
#pragma unroll
        for (int ks = 0; ks < BD / 16; ++ks) acc[ks % DT] = T::mfma(at[ks], db[ks / DT], acc[ks % DT]);
      }
      if (DS) {
#pragma unroll
        for (int ks = 0; ks < BD / 16; ++ks) dp = T::mfma(ar[ks], kv_op[ks], dp);
      }
      if (ldw) put_ld((s + 2) & (NB - 1));
      phase_end();
      advance(h_ahd, t_ahd);
    };
    if (nsteps > 0) {
      step(0, U{}, F{});
      for (int s = 1; s < nsteps; ++s) step(s, U{}, U{});
      step(nsteps, F{}, U{});
    }
  }
  if (key < klim) {
    if (dswave)
      store_t<T, BD>((uint16_t*)p.dk + (int64_t)b * p.dk_sb + (int64_t)hkv * p.dk_sh + (int64_t)koff * p.dk_ss, p.dk_ss,
                     key, acc, p.scale);
    else
      store_t<T, BD>((uint16_t*)p.dv + (int64_t)b * p.dv_sb + (int64_t)hkv * p.dv_sh + (int64_t)koff * p.dv_ss, p.dv_ss,
                     key, acc, 1.f);
  }
}

template <class T, int BD, bool CAUSAL, bool MASK, bool PK>
__global__ __launch_bounds__(64 * NWQ, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int DT = BD / 32;   // 32-wide d tiles
  constexpr int CPR = BD / 8;   // 16-byte chunks per tile row
  constexpr int NPQ = BD / 64;  // copy instructions per wave and tile (a quarter tile)
  // Three slots of the K and V tiles (K read both ways, V by rows).
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[3][2][TR * BD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 31, h = lane >> 5;
  // Workgroups in order of decreasing work (under the causal mask the last
  // query blocks see the most keys), the (batch, head) index fastest.
  const int lin = blockIdx.x + blockIdx.y * gridDim.x, nbh = p.B * p.Hq;
  const int bh = lin % nbh, b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.G;
  const int q0 = (CAUSAL ? (int)gridDim.x - 1 - lin / nbh : lin / nbh) * BLKQ;
  const int qi = q0 + 32 * w + c;  // this lane's query row (column of S^T)
  int Lq, Lk, qoff, koff;
  batch_geometry<PK>(p, b, Lq, Lk, qoff, koff);
  // A packed batch's row block past its rows has nothing to compute or write.
  if (PK && q0 >= Lq) return;
  const int rlim = PK ? Lq : p.Sq;  // rows the lanes load and store
  const int klim = PK ? Lk : p.Skv;  // keys the tile copies may read
  const int diag = Lk - Lq;
  // mask bytes of the lane's query row (read only where qi < Sq)
  const uint8_t* mq = MASK ? p.mask + (int64_t)b * p.m_sb + (int64_t)hq * p.m_sh + (int64_t)qi * p.m_ss : nullptr;
  const uint16_t* qg = (const uint16_t*)p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)qoff * p.q_ss;
  const uint16_t* dg = (const uint16_t*)p.dout + (int64_t)b * p.do_sb + (int64_t)hq * p.do_sh + (int64_t)qoff * p.do_ss;
  const uint16_t* kg = (const uint16_t*)p.k + (int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh + (int64_t)koff * p.k_ss;
  const uint16_t* vg = (const uint16_t*)p.v + (int64_t)b * p.v_sb + (int64_t)hkv * p.v_sh + (int64_t)koff * p.v_ss;
  u32x4 qop[BD / 16], dop[BD / 16];
  load_bop<BD>(qop, qg, p.q_ss, min(qi, rlim - 1));
  load_bop<BD>(dop, dg, p.do_ss, min(qi, rlim - 1));
  // S^T and dP^T start from -LSE / scale and -Delta of the lane's row, so
  // that P = exp2(S^T scale log2e) and dS^T = P dP^T; padding rows and rows
  // without keys start from +inf (their elements are masked).
  // Delta_i = dO_i . O_i in fp32 (from O + o_lo, the unrounded output, when
  // the forward wrote its rounding residual: the precise dpsum of the
  // sparse-MLA page): the lane's half of row qi's columns, the columns of its
  // dO operands, then the two halves summed. It is stored for the dK/dV
  // kernel, which runs after this one.
  const int qc = min(qi, rlim - 1);
  const uint16_t* og =
      (const uint16_t*)p.o + (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)(qoff + qc) * p.o_ss;
  float dacc = 0.f;
#pragma unroll
  for (int ks = 0; ks < BD / 16; ++ks) {
    const u32x4 ov = *(const u32x4*)(og + 16 * ks + 8 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) dacc = T::dot2(ov[e], dop[ks][e], dacc);
  }
  if (p.o_lo) {
    const float* lo = p.o_lo + (int64_t)b * p.ol_sb + (int64_t)hq * p.ol_sh + (int64_t)(qoff + qc) * p.ol_ss;
#pragma unroll
    for (int ks = 0; ks < BD / 16; ++ks) {
      const float4 l0 = *(const float4*)(lo + 16 * ks + 8 * h), l1 = *(const float4*)(lo + 16 * ks + 8 * h + 4);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 dd = T::unpack2(dop[ks][e]);
        dacc = __builtin_fmaf(dd[0], lv[2 * e], dacc);
        dacc = __builtin_fmaf(dd[1], lv[2 * e + 1], dacc);
      }
    }
  }
  const float delta = half_sum(dacc);
  if (h == 0 && qi < rlim) p.delta[ld_index<PK>(p, b, hq, qoff, qi)] = delta;
  float s_init = INFINITY, d_init = 0.f;
  if (qi < Lq) {
    const float l = p.lse[ld_index<PK>(p, b, hq, qoff, qi)];
    s_init = l == -INFINITY ? INFINITY : -l / p.scale;
    d_init = -delta;
  }
  f32x16 dq_t[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_t[dt][i] = 0.f;
  // Keys any row of this block sees: j <= q0 + BLKQ - 1 + diag (causal).
  const int kend = q0 >= Lq ? 0 : CAUSAL ? max(0, min(Lk, q0 + BLKQ + diag)) : Lk;
  const int nkt = (kend + TR - 1) / TR;
  // K and V tiles: a three-deep LDS ring (slot t % 3) filled by LDS-DMA two
  // tiles ahead: wave w copies a quarter of tile t + 2 (K for w < 4, V for
  // w >= 4; chunk positions 64 (NPQ (w % 4) + n) + lane, n < NPQ) at the
  // start of step t into the slot of tile t - 1 (every wave passed the
  // barrier that ended its step), and waits for its copies of tile t + 1 at
  // the end of step t. Rows at or past Skv fetch row Skv - 1.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const bool c_v = wu >= 4;
  int crow[NPQ];
  uint32_t cchunk[NPQ];
#pragma unroll
  for (int n = 0; n < NPQ; ++n) {
    const int pos = 64 * (NPQ * (wu & 3) + n) + lane, row = pos / CPR;
    crow[n] = row;
    cchunk[n] = (uint32_t)(bsw<BD>(row, pos % CPR) * 16);
  }
  const int64_t c_ss = c_v ? p.v_ss : p.k_ss;
  const uint16_t* c_head = c_v ? vg : kg;
  const uint32_t c_rb = (uint32_t)c_ss * 2u;
  const uint32_t c_lds = lds_addr_of(sbuf[0][c_v ? 1 : 0]) + (wu & 3) * (NPQ * 1024);
  auto dma = [&](int t, int sl) __attribute__((always_inline)) {
    const int j0 = t * TR;
    const uint16_t* base = c_head + (int64_t)j0 * c_ss;
    const int rmax = klim - 1 - j0;
    const uint32_t l0 = c_lds + (uint32_t)sl * (2 * TR * BD * 2);
#pragma unroll
    for (int n = 0; n < NPQ; ++n) lds_copy16(base, (uint32_t)min(crow[n], rmax) * c_rb + cchunk[n], l0 + n * 1024);
  };
  if (nkt > 0) {
    dma(0, 0);
    if (nkt > 1) {
      dma(1, 1);
      wait_vmem_below<NPQ>();
    } else {
      wait_vmem();
    }
  }
  int sl = 0;  // slot of tile t
  for (int t = 0; t < nkt; ++t) {
    const int j0 = t * TR;
    // Tile t is in LDS and every wave is done with tile t - 1.
    barrier_keep_copies();
    if (t + 2 < nkt) dma(t + 2, sl == 0 ? 2 : sl - 1);
    const uint16_t* sKr = sbuf[sl][0];
    const uint16_t* sKt = sKr;
    const uint16_t* sVr = sbuf[sl][1];
    // Two waves share each SIMD here (the register budget is 256), so the
    // operands are read as the MFMAs consume them.
    f32x16 s0, dp0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = s_init;
      dp0[i] = d_init;
    }
#pragma unroll
    for (int ks = 0; ks < BD / 16; ++ks) {
      s0 = T::mfma(row_op<BD>(sKr, ks), qop[ks], s0);
      dp0 = T::mfma(row_op<BD>(sVr, ks), dop[ks], dp0);
    }
    // Element i: key j0 + r, r = 8 (i / 4) + 4 h + i % 4; query row qi.
    // A block whose keys all exist and are seen by every row of the wave
    // needs no per-element test.
    const int qw0 = q0 + 32 * w;
    const bool inside = !MASK && __builtin_amdgcn_readfirstlane(
                                     (j0 + TR <= Lk && qw0 + 31 < Lq && (!CAUSAL || j0 + 31 <= qw0 + diag)) ? 1 : 0);
    f32x16 dsm;
    if (inside) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dsm[i] = fast_exp2(s0[i] * p.scale_log2) * dp0[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = j0 + 8 * (i >> 2) + 4 * h + (i & 3);
        bool ok = kj < Lk && qi < Lq;
        if (CAUSAL) ok = ok && kj <= qi + diag;
        if (MASK) ok = ok && mq[kj] == 0;
        dsm[i] = ok ? fast_exp2(s0[i] * p.scale_log2) * dp0[i] : 0.f;
      }
    }
#pragma unroll
    for (int ks = 0; ks < TR / 16; ++ks) {
      const u32x4 db = pack_b<T>(dsm, ks);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dq_t[dt] = T::mfma(tr_op<BD>(sKt, dt, ks), db, dq_t[dt]);
    }
    // this wave's copies of tile t + 1 are complete (tile t + 2 may fly)
    if (t + 2 < nkt)
      wait_vmem_below<NPQ>();
    else
      wait_vmem();
    sl = sl == 2 ? 0 : sl + 1;
  }
  if (qi < rlim)
    store_t<T, BD>((uint16_t*)p.dq + (int64_t)b * p.dq_sb + (int64_t)hq * p.dq_sh + (int64_t)qoff * p.dq_ss, p.dq_ss, qi,
                   dq_t, p.scale);
}

// Delta_i = dO_i . O_i (or dO_i . (O_i + o_lo_i)) in fp32 for every row the
// dK/dV kernel reads, ahead of it, with the per-tile records of its
// accumulator start values (the dS-store path; the other path forms Delta in
// its dQ kernel and the dK/dV kernel loads LSE and Delta itself). BD / 8
// consecutive lanes share a row, 8 columns each.
template <class T, int BD, bool PK>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = BD / 8;     // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per workgroup
  const int bh = blockIdx.y, b = bh / p.Hq, hq = bh % p.Hq;
  int Lq, Lk, qoff, koff;
  batch_geometry<PK>(p, b, Lq, Lk, qoff, koff);
  const int rlim = PK ? Lq : p.Sq;
  const int rlim32 = (rlim + TR - 1) & ~(TR - 1);  // rows of the batch's start-value records
  if ((int)blockIdx.x * RPB >= rlim32) return;
  const int sub = threadIdx.x % LPR, i = blockIdx.x * RPB + threadIdx.x / LPR;
  const int ic = min(i, rlim - 1);
  const u32x4 ov = *(const u32x4*)((const uint16_t*)p.o + (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh +
                                   (int64_t)(qoff + ic) * p.o_ss + 8 * sub);
  const u32x4 dv = *(const u32x4*)((const uint16_t*)p.dout + (int64_t)b * p.do_sb + (int64_t)hq * p.do_sh +
                                   (int64_t)(qoff + ic) * p.do_ss + 8 * sub);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = T::dot2(ov[e], dv[e], acc);
  if (p.o_lo) {
    const float* lo = p.o_lo + (int64_t)b * p.ol_sb + (int64_t)hq * p.ol_sh + (int64_t)(qoff + ic) * p.ol_ss + 8 * sub;
    const float4 l0 = *(const float4*)lo, l1 = *(const float4*)(lo + 4);
    const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 dd = T::unpack2(dv[e]);
      acc = __builtin_fmaf(dd[0], lv[2 * e], acc);
      acc = __builtin_fmaf(dd[1], lv[2 * e + 1], acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (sub == 0 && i < rlim) p.delta[ld_index<PK>(p, b, hq, qoff, i)] = acc;
  // The dK/dV kernel's start values of S (-LSE / scale; +inf for rows
  // without keys and past the batch, whose elements it masks) and of dP
  // (-Delta).
  if (sub == 0 && i < rlim32) {
    float* rec = p.ldrec + ((int64_t)(b * p.Hq + hq) * (p.ds_qp / TR) + i / TR) * (2 * TR) + i % TR;
    const float l = i < rlim ? p.lse[ld_index<PK>(p, b, hq, qoff, i)] : -INFINITY;
    rec[0] = l == -INFINITY ? INFINITY : l * (-1.f / p.scale);
    rec[TR] = -(i < rlim ? acc : 0.f);
  }
}

// dQ = scale dS K from the dS the dK/dV kernel stored: a workgroup of 8
// waves owns 256 query rows of one head (32 per wave) and sweeps the 32-key
// tiles its rows see. Per tile, the K tile (32 x D) and the 16 KB of dS
// blocks of the 256 rows (contiguous in the workspace) come by LDS DMA into
// a six-deep ring five tiles ahead; dQ^T += K^T dS^T takes both operands
// through transposing reads, K^T as in the recomputing dQ kernel and the
// wave's own 32 x 32 dS block (64 bytes per key, so the four keys of a
// transposing read span all banks) in the same key order. The block holds
// row 8 ((p % 16) / 4) + 4 (p / 16) + p % 4 at position p, so accumulator
// column n (the lane's) is that row for p = n. A wave skips the
// tiles none of its rows sees (the dK/dV kernel did not write them); masked
// and padded elements were stored as zeros.
template <class T, int BD, bool CAUSAL, bool PK>
__global__ __launch_bounds__(64 * NWQ, 1) void bwd_dqg_kernel(BwdParams p) {
  constexpr int DT = BD / 32;
  constexpr int CK = 4 * BD;           // 16-byte chunks of a K tile (32 rows x BD)
  constexpr int CS = 32 * BLKQ / 8;    // chunks of a dS^T tile (32 keys x 256 rows)
  constexpr int NI = (CK + CS) / 64;   // wave copy instructions per tile (8 waves share them)
  constexpr int SLOT = (CK + CS) * 8;  // 16-bit elements per ring slot
  constexpr int NS = 6;                // ring slots (tiles t + 1 .. t + NS - 1 in flight)
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[NS][SLOT];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 31, h = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int lin = blockIdx.x + blockIdx.y * gridDim.x, nbh = p.B * p.Hq;
  const int bh = lin % nbh, b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.G;
  const int q0 = (CAUSAL ? (int)gridDim.x - 1 - lin / nbh : lin / nbh) * BLKQ;
  int Lq, Lk, qoff, koff;
  batch_geometry<PK>(p, b, Lq, Lk, qoff, koff);
  if (PK && q0 >= Lq) return;
  const int rlim = PK ? Lq : p.Sq;
  const int klim = PK ? Lk : p.Skv;
  const int diag = Lk - Lq;
  const int kend = q0 >= Lq ? 0 : CAUSAL ? max(0, min(Lk, q0 + BLKQ + diag)) : Lk;
  const int nkt = (kend + TR - 1) / TR;
  const uint16_t* kg = (const uint16_t*)p.k + (int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh + (int64_t)koff * p.k_ss;
  const uint16_t* dsg = p.ds + ((int64_t)(b * p.Hq + hq) * p.ds_nrb + (q0 >> 8)) * p.ds_nkt * (8 * 1024);
  // This wave's copy instructions: u = w, w + 8, w + 16 (< NI); u < CK / 64
  // copies K chunks 64 u + lane, the others dS^T chunks.
  uint32_t coff[3];
  bool cisk[3];
  int crow[3];
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int u = wu + 8 * n, pos = 64 * u + lane;
    cisk[n] = u < CK / 64;
    if (cisk[n]) {
      const int row = pos / (BD / 8);
      crow[n] = row;
      coff[n] = (uint32_t)(bsw<BD>(row, pos % (BD / 8)) * 16);
    } else {
      crow[n] = 0;
      coff[n] = (uint32_t)(pos - CK) * 16u;
    }
  }
  const int ncw = (NI - wu + 7) / 8;  // copy instructions of this wave per tile
  const uint32_t k_rb = (uint32_t)p.k_ss * 2u;
  const uint32_t l_base = lds_addr_of(sbuf[0]);
  auto dma = [&](int t, int sl) __attribute__((always_inline)) {
    const int j0 = t * TR;
    const uint32_t l0 = l_base + (uint32_t)sl * (SLOT * 2);
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int u = wu + 8 * n;
      if (u < NI) {
        if (cisk[n])
          lds_copy16(kg + (int64_t)j0 * p.k_ss, (uint32_t)min(crow[n], klim - 1 - j0) * k_rb + coff[n], l0 + u * 1024);
        else
          lds_copy16(dsg + (int64_t)t * (8 * 1024), coff[n], l0 + u * 1024);
      }
    }
  };
  // Waits for the oldest tile in flight while NS - 2 later ones may still
  // fly (all of them near the end of the sweep).
  auto wait_tile = [&](bool keep_next) __attribute__((always_inline)) {
    if (!keep_next)
      wait_vmem();
    else if (ncw == 3)
      wait_vmem_below<3 * (NS - 2)>();
    else
      wait_vmem_below<2 * (NS - 2)>();
  };
  for (int t = 0; t < NS - 1 && t < nkt; ++t) dma(t, t);
  if (nkt > 0) wait_tile(nkt >= NS - 1);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  const int qw0 = q0 + 32 * wu;
  // transposing reads of the wave's dS block: keys 16 ks + 4 h + (lane &
  // 15) / 4 and +8, positions 16 ((lane >> 4) & 1) + 4 (lane & 3) .. +3
  const int vrow = 4 * h + ((lane & 15) >> 2);
  const int col = 1024 * wu + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int sl = 0;
  for (int t = 0; t < nkt; ++t) {
    const int j0 = t * TR;
    barrier_keep_copies();
    // into the slot of tile t - 1, which every wave has finished
    if (t + NS - 1 < nkt) dma(t + NS - 1, sl == 0 ? NS - 1 : sl - 1);
    const bool active = qw0 < Lq && (!CAUSAL || j0 <= qw0 + 31 + diag);
    if (active) {
      const uint16_t* sK = sbuf[sl];
      const uint16_t* sS = sbuf[sl] + CK * 8;
#pragma unroll
      for (int ks = 0; ks < TR / 16; ++ks) {
        const int r0 = 16 * ks + vrow, r1 = r0 + 8;
        const u32x2 lo = lds_read_tr16(sS + col + r0 * 32);
        const u32x2 hi = lds_read_tr16(sS + col + r1 * 32);
        const u32x4 bop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = T::mfma(tr_op<BD>(sK, dt, ks), bop, acc[dt]);
      }
    }
    wait_tile(t + NS - 1 < nkt);
    sl = sl == NS - 1 ? 0 : sl + 1;
  }
  const int qi = qw0 + 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3);
  if (qi < rlim)
    store_t<T, BD>((uint16_t*)p.dq + (int64_t)b * p.dq_sb + (int64_t)hq * p.dq_sh + (int64_t)qoff * p.dq_ss, p.dq_ss, qi,
                   acc, p.scale);
}

template <class T, int BD, bool CAUSAL, bool MASK, bool PK = false>
hipError_t launch_bwd_t(BwdParams& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  const dim3 gq((unsigned)((p.Sq + BLKQ - 1) / BLKQ), (unsigned)(p.B * p.Hq));
  const dim3 gk((unsigned)((p.Skv + BLK - 1) / BLK), (unsigned)(p.B * p.Hkv));
  const bool keys = p.Skv > 0 && p.B * p.Hkv > 0;
  if (p.ds) {
    // Delta, then dK / dV storing dS, then dQ from dS.
    if (rows > 0) {
      constexpr int RPB = 256 / (BD / 8);
      hipLaunchKernelGGL((bwd_delta_kernel<T, BD, PK>), dim3((unsigned)((p.ds_qp + RPB - 1) / RPB), (unsigned)(p.B * p.Hq)),
                         dim3(256), 0, st, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (keys) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, BD, CAUSAL, MASK, PK, true>), gk, dim3(512), 0, st, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (rows > 0) hipLaunchKernelGGL((bwd_dqg_kernel<T, BD, CAUSAL, PK>), gq, dim3(64 * NWQ), 0, st, p);
    return hipGetLastError();
  }
  // The dQ kernel also writes Delta, which the dK/dV kernel reads.
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, BD, CAUSAL, MASK, PK>), gq, dim3(64 * NWQ), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (keys) hipLaunchKernelGGL((bwd_dkdv_kernel<T, BD, CAUSAL, MASK, PK, false>), gk, dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace

template <class T, int BD>
hipError_t launch_bwd_m(bool causal, bool mask, BwdParams& p, hipStream_t st) {
  if (mask) return causal ? launch_bwd_t<T, BD, true, true>(p, st) : launch_bwd_t<T, BD, false, true>(p, st);
  return causal ? launch_bwd_t<T, BD, true, false>(p, st) : launch_bwd_t<T, BD, false, false>(p, st);
}

template <class T, int BD>
hipError_t launch_bwd_pk(bool causal, BwdParams& p, hipStream_t st) {
  return causal ? launch_bwd_t<T, BD, true, false, true>(p, st) : launch_bwd_t<T, BD, false, false, true>(p, st);
}

hipError_t launch_bwd_varlen(Dt dt, int d, bool causal, BwdParams& p, hipStream_t stream) {
  if (dt == Dt::BF16)
    return d == 64 ? launch_bwd_pk<BF16, 64>(causal, p, stream) : launch_bwd_pk<BF16, 128>(causal, p, stream);
  return d == 64 ? launch_bwd_pk<F16, 64>(causal, p, stream) : launch_bwd_pk<F16, 128>(causal, p, stream);
}

hipError_t launch_bwd(Dt dt, int d, bool causal, bool mask, BwdParams& p, hipStream_t stream) {
  if (dt == Dt::BF16)
    return d == 64 ? launch_bwd_m<BF16, 64>(causal, mask, p, stream) : launch_bwd_m<BF16, 128>(causal, mask, p, stream);
  return d == 64 ? launch_bwd_m<F16, 64>(causal, mask, p, stream) : launch_bwd_m<F16, 128>(causal, mask, p, stream);
}

}  // namespace fa
