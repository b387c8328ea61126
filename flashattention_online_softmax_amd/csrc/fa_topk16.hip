// Top-k gathered sparse MLA forward for gfx950 (one KV head shared by every
// query head), fp16 / bf16, Dqk = 576 (512 latent + 64 rope), Dv = 512.
//
// Method: per token t, attention of every query head over the keys named in
// idx[t, :] (the sparse-MLA forward of the flash-attention SM100 page,
// background section), with that page's exact running max (threshold 0: any
// growth of a row max rescales O and l, so the largest p of a row is exactly
// 1.0 before it is rounded for P.V). The online-softmax recurrence is the one
// of the "FlashAttention correctness verification" page (tiled computation,
// loop invariant).
//
// This file is compiled into the run-time loaded code object (see build.py):
// a wave keeps its O^T accumulators in all 256 AGPRs next to about 230
// VGPRs, a split the code object gets through amdgpu-agpr-alloc.
//
// Decomposition (MI355X): one workgroup of 4 waves (one per SIMD) per token
// and 128 query heads; wave w owns heads 32 w .. 32 w + 31 as two 16-head
// tiles. The MFMAs are v_mfma_f32_16x16x32; every K or V operand read from
// LDS feeds both head tiles. Q^T (576 x 32) stays in VGPRs as the B operand
// of S^T = K_g Q^T; O^T (512 x 32 fp32) fills the AGPRs. The valid entries
// of idx[t, :] are compacted into LDS (list order kept, negative slots
// dropped); 32 consecutive list entries form a tile whose key rows (1152
// bytes each) are gathered from HBM/L2 straight into LDS by
// global_load_lds_dwordx4 (no register staging; an index at or past S reads
// the last row). When V is the first 512 columns of K (the MLA latent) the
// tiles live in a 4-deep ring and P.V reads V^T out of the gathered K rows
// with ds_read_b64_tr_b16; otherwise K and V tiles have 2-deep rings of their
// own. Only the last list tile can be partial: its padding rows repeat a
// valid key and their scores are masked to -inf. Tiles are visited first,
// last, then the rest in list order (see visit()).
//
// Lane l of a wave (G = l / 16, n = l % 16) owns heads 16 ht + n of the wave
// (ht = 0, 1) and, of each 32-key tile, keys 4 G .. 4 G + 3 and
// 16 + 4 G .. 16 + 4 G + 3: the S^T accumulator layout of the 16x16x32 MFMA,
// which is also the key order of its B operand when P^T is packed in-lane.
// The row max and row sum are in-lane reductions plus two lane swaps.
//
// Per visited tile j a wave runs two MFMA phases:
//   1. S^T(j+1) = K_{j+1} Q^T (72 MFMAs, VGPR accumulators) while its VALU
//      does the softmax of tile j; when a row max grew, the O^T tiles of its
//      16-head tile are rescaled;
//   2. O^T += V_j^T P_j^T (64 MFMAs, AGPR accumulators) while its VALU
//      computes the gather offset of the next tile copy;
// then it waits for its share of tile j+2's copies, passes the workgroup
// barrier and starts the copy of tile j+4 into the slot tile j leaves.
#include <stdint.h>

#include "fa_asm.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int TB = 32;                           // gathered keys per tile
constexpr int NWAVE = 4;
constexpr int CHK = DQK / 8;                     // 16-byte chunks per K row (72)
constexpr int CHV = DV / 8;                      // ... per V row (64)
constexpr int KCOPY = CHK / 8;                   // copy instructions per wave per K tile (9)
constexpr int KSTEP = DQK / 32;                  // MFMA k-steps of S^T (18)
constexpr int NKOP = 2 * KSTEP;                  // K operands per tile (2 key halves x 18)
constexpr int NDT = DV / 16;                     // 16-row d tiles of O^T (32)
constexpr uint32_t KTILE = TB * DQK * 2;         // bytes of a K tile
constexpr uint32_t VTILE = TB * DV * 2;          // bytes of a V tile
constexpr int LIST = 4096;                       // longest index row
constexpr int NOPS = NKOP + DV / 16;             // LDS operands per step: 36 K, then 32 V
constexpr int AHEAD = 6, RING = 8;               // operands read ahead / their ring
// Operand u >= NOPS of a step of parity par is operand u - NOPS of the next
// step (parity par ^ 1) in the same ring slot.
static_assert((2 * NOPS) % RING == 0, "slot(par, u + NOPS) == slot(par ^ 1, u)");
constexpr int EXP_GAPS = 8;                      // phase-1 MFMAs carrying the exponentials (a pair each)
constexpr int PREP_AT = 48;                      // phase-2 MFMA after which the next gather offset is read

static_assert(TB == 8 * NWAVE, "each wave copies 8 rows of a tile");
static_assert(EXP_GAPS == 8, "8 score pairs per lane (2 head tiles x 2 key halves x 2)");

// A ring slot holds a tile as 4 regions of 8 rows (RK bytes for K rows,
// RV for V rows); region byte 1024 g + 128 r + 16 e is position e of the
// 8-chunk group g of row r. Position e of row r in region w holds logical
// chunk e ^ rsw(r, w) of its group, rsw(r, w) = (r >> 1) | 4 (w % 2): over
// the 16 rows 0..15 (or 16..31) of a tile the pair (r % 2, rsw) takes 16
// distinct values. Measured on gfx950 (per-pattern LDS microbenchmark), the
// K operand reads (ds_read_b128, 16 rows x one chunk per 16 lanes) then see
// no bank conflicts and run at ~200 B/clk per CU, while the transposed V^T
// reads (4 rows x 32 bytes per 16 lanes) run at ~87 B/clk; the alternative
// (r & 6) | (w % 2), conflict-free for the V^T reads on paper, halves the K
// read rate and does not speed up the V^T reads.
constexpr uint32_t RK = 8 * DQK * 2;  // 9216
constexpr uint32_t RV = 8 * DV * 2;   // 8192
__device__ __forceinline__ int rsw(int r, int w) { return (r >> 1) | ((w & 1) << 2); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32 with the accumulator file chosen here: lane l holds
// A[m = l % 16][k = 8 (l / 16) + e], B[k = 8 (l / 16) + e][n = l % 16] and
// D[m = 4 (l / 16) + i][n = l % 16].
template <class T>
struct Mma16;
template <>
struct Mma16<BF16> {
  static __device__ __forceinline__ void v0(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void v(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void a(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
};
template <>
struct Mma16<F16> {
  static __device__ __forceinline__ void v0(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void v(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void a(f32x4& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
};

// Maximum / sum over the 4 lanes l % 16 + 16 G (G = 0..3) that hold one head:
// v_permlane16_swap pairs l with l ^ 16, v_permlane32_swap l with l ^ 32 (with
// both operands x, element 0 / 1 of the result hold own / partner values).
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return half_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return half_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Waits until at most n (0, KCOPY or 2 KCOPY) copies of this wave are in
// flight; n is wave-uniform.
__device__ __forceinline__ void wait_copies_below(int n) {
  if (n >= 2 * KCOPY)
    wait_vmem_below<2 * KCOPY>();
  else if (n >= KCOPY)
    wait_vmem_below<KCOPY>();
  else
    wait_vmem();
}

// Wait states between VALU writes of an accumulator tile and the MFMA that
// reads it next; the writes are placed before this point.
__device__ __forceinline__ void acc_written4(f32x4& a) { asm volatile("s_nop 4" : "+a"(a)); }

template <class T, bool VALIAS>
__device__ __forceinline__ void topk16_body(const TopkParams& p) {
  using Mm = Mma16<T>;
  constexpr int KR = VALIAS ? 4 : 2;  // K tile ring depth
  constexpr uint32_t V_BASE = KR * KTILE;
  constexpr uint32_t L_BASE = V_BASE + (VALIAS ? 0u : 2u * VTILE);
  __shared__ __attribute__((aligned(16))) uint8_t s_mem[L_BASE + LIST * 4];
  int* const s_list = (int*)(s_mem + L_BASE);
  int* const s_wcount = (int*)s_mem;  // scan scratch; the ring is not in use yet
  const uint32_t lds0 = lds_addr_of(s_mem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, n = lane & 15;
  // Tokens in decreasing order: under a causal index pattern the late tokens
  // have the longest lists and start first.
  const int tb = (int)blockIdx.x / p.n_htiles;
  const int t = p.T - 1 - tb;
  const int head0 = ((int)blockIdx.x - tb * p.n_htiles) * 128 + w * 32;
  const bool active = head0 < p.Hq;

  // The index row first, into registers (thread tid owns the slots
  // [tid*spt, tid*spt + spt), spt <= 16): the compaction below then waits
  // for it alone, while the Q loads issued after it are still in flight.
  const int32_t* irow = p.idx + (int64_t)t * p.idx_st;
  const int spt = (p.W + 255) / 256;
  int iv[16];
  if (spt == 8 && p.W == 2048 && (((uintptr_t)irow) & 15) == 0) {
    const int4 a = *(const int4*)(irow + tid * 8);
    const int4 b = *(const int4*)(irow + tid * 8 + 4);
    iv[0] = a.x; iv[1] = a.y; iv[2] = a.z; iv[3] = a.w;
    iv[4] = b.x; iv[5] = b.y; iv[6] = b.z; iv[7] = b.w;
#pragma unroll
    for (int e = 8; e < 16; ++e) iv[e] = -1;
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int s = tid * spt + e;
      iv[e] = (e < spt && s < p.W) ? irow[s] : -1;
    }
  }
  asm volatile("" ::: "memory");  // keep the Q loads behind the index loads

  // Q^T operands (B operand of S^T): qop[ht][ks] = Q[t, head 16 ht + n,
  // 32 ks + 8 G .. +7]. Query heads are padded to the wave's 32: a head at or
  // past Hq computes on head Hq - 1 and stores nothing (a wave past Hq
  // entirely stores nothing at all).
  u32x4 qop[2][KSTEP];
  {
    const uint16_t* qt = (const uint16_t*)p.q + (int64_t)t * p.q_st + 8 * G;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hh = min(head0 + 16 * ht + n, p.Hq - 1);
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) qop[ht][ks] = *(const u32x4*)(qt + (int64_t)hh * p.q_sh + 32 * ks);
    }
  }

  // Compact the valid indices of row t into s_list (list order kept).
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) cnt += iv[e] >= 0 ? 1 : 0;
  int incl = cnt;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wcount[w] = incl;
  __syncthreads();
  int off = incl - cnt;
  for (int ww = 0; ww < w; ++ww) off += s_wcount[ww];
  const int n_valid = __builtin_amdgcn_readfirstlane(s_wcount[0] + s_wcount[1] + s_wcount[2] + s_wcount[3]);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (iv[e] >= 0) s_list[off++] = iv[e];
  __syncthreads();
  const int n_tiles = (n_valid + TB - 1) / TB;
  // Retire the Q loads here, visibly to the compiler, before any copy is in
  // flight: its wait for them would otherwise stay inside the loop and, as
  // the copies count on the same counter, also wait for every copy.
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) asm volatile("" ::"v"(qop[ht][ks]));

  // Gathers. Wave w copies rows 8 w .. 8 w + 7 of a tile into its region of
  // the ring slot; lane l handles row 8 w + l / 8. Copy instruction g (one
  // per 8-chunk group of a row) fills region bytes 1024 g + 16 l, which hold
  // the row's logical chunk 8 g + (l % 8 ^ rsw(l / 8, w)).
  const uint32_t krow = (uint32_t)p.k_ss * 2u;
  const uint32_t vrow = (uint32_t)p.v_ss * 2u;
  const uint32_t s_rows = (uint32_t)p.S;
  const int crow = lane >> 3;
  const uint32_t cchunk = (uint32_t)(((lane & 7) ^ rsw(crow, w)) << 4);
  // Byte offset of a key row (an index past the last row reads the last row).
  // Visit order of the list tiles: the first, the last, then the others in
  // list order. Index lists tend to hold their strongest key at one end (an
  // indexer ranks keys best first; a causal list in key order ends with the
  // token's own key), and meeting each row's maximum early makes later
  // growth, each of which costs an exact rescale of O, rare. The running max
  // stays exact in any order; only the rounding order of the sums changes.
  auto visit = [&](int step) __attribute__((always_inline)) {
    return step == 0 ? 0 : step == 1 ? n_tiles - 1 : step - 1;
  };
  // Gather offset of this lane's key row of the tile visited at `step` (steps
  // past the last one read a valid row and are never used).
  auto gather_base = [&](int step, uint32_t row_bytes) __attribute__((always_inline)) {
    const uint32_t key = (uint32_t)s_list[min(visit(step) * TB + 8 * w + crow, n_valid - 1)];
    return min(key, s_rows - 1) * row_bytes + cchunk;
  };
  uint32_t kbase;  // gather offset (group 0) of the next K copy
  auto prep_k = [&](int step) __attribute__((always_inline)) { kbase = gather_base(step, krow); };
  auto issue_k = [&](int step) __attribute__((always_inline)) {
    const uint32_t l0 = lds0 + (uint32_t)(step % KR) * KTILE + (uint32_t)w * RK;
#pragma unroll
    for (int g = 0; g < KCOPY; ++g) lds_copy16(p.k, kbase + 128u * g, l0 + 1024u * g);
  };
  auto issue_v = [&](int step) __attribute__((always_inline)) {
    const uint32_t vb = gather_base(step, vrow);
    const uint32_t l0 = lds0 + V_BASE + (uint32_t)(step & 1) * VTILE + (uint32_t)w * RV;
#pragma unroll
    for (int g = 0; g < CHV / 8; ++g) lds_copy16(p.v, vb + 128u * g, l0 + 1024u * g);
  };

  // K operand r = 2 ks + kt (A operand of S^T, key half kt, k-step ks): row
  // 16 kt + n (region 2 kt + n / 8, row n % 8), logical chunk 4 ks + G (group
  // ks / 2, position (4 (ks % 2) + G) ^ rsw), at byte
  // koff[ks % 2] + 2 RK kt + 1024 (ks / 2) of the slot.
  uint32_t koff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    koff[par] = (uint32_t)((n >> 3) * RK + (n & 7) * 128 + (((4 * par + G) ^ rsw(n & 7, n >> 3)) << 4));
  auto kread = [&](uint32_t tile_addr, int r) __attribute__((always_inline)) -> u32x4 {
    const int kt = r & 1, ks = r >> 1;
    const int imm = (kt * 2 * RK + (ks >> 1) * 1024) / 2;
    return *(const __attribute__((address_space(3))) u32x4*)(lds_ptr(tile_addr + koff[ks & 1]) + imm);
  };
  // V^T operand dt (A operand of O^T += V^T P^T: d rows 16 dt + n, keys in
  // the order of P^T), two ds_read_b64_tr_b16: lane l reads 4 consecutive
  // elements of row vr (low half) or vr + 16 (high half) at column
  // 16 dt + vc. Row vr is row vr % 8 of region vr / 8 (= G / 2); column
  // 16 dt + vc is in logical chunk 2 dt + vc / 8 (group dt / 4). voff[dt % 4]
  // + 1024 (dt / 4) is the low half's byte offset in the slot, + 2 RB the high
  // half's.
  constexpr uint32_t RB = VALIAS ? RK : RV;
  const int vr = 4 * G + ((lane & 15) >> 2);
  const int vc = 4 * (lane & 3);
  uint32_t voff[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4)
    voff[d4] = (uint32_t)((G >> 1) * RB + (vr & 7) * 128 + (((2 * d4 + (vc >> 3)) ^ rsw(vr & 7, G >> 1)) << 4) +
                          2 * (vc & 7));
  auto vread = [&](uint32_t tile_addr, int dt) __attribute__((always_inline)) -> u32x4 {
    const int imm = ((dt >> 2) * 1024) / 2;
    const u32x2 lo = lds_read_tr16(lds_ptr(tile_addr + voff[dt & 3]) + imm);
    const u32x2 hi = lds_read_tr16(lds_ptr(tile_addr + voff[dt & 3]) + imm + RB);
    const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return v;
  };
  auto ktile = [&](int step) __attribute__((always_inline)) { return lds0 + (uint32_t)(step % KR) * KTILE; };
  auto vtile = [&](int step) __attribute__((always_inline)) {
    return VALIAS ? ktile(step) : lds0 + V_BASE + (uint32_t)(step & 1) * VTILE;
  };

  // O^T accumulator tiles oacc[dt][ht]: d rows 16 dt + 4 G + i, head 16 ht + n.
  f32x4 oacc[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      oacc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_written4(oacc[dt][ht]);  // O^T lives in AGPRs from here on
    }
  float m_run[2] = {-INFINITY, -INFINITY};  // running row max (exp2 domain)
  float l_run[2] = {0.f, 0.f};              // row sum over this lane's keys
  float alpha[2] = {1.f, 1.f};
  u32x4 pop[2];                             // P^T operands of the tile between phases
  f32x4 s0[2][2], s1[2][2];                 // [kt][ht] score tiles, alternately S(j), S(j+1)

  // The LDS operands of a step, u = 0 .. NOPS-1 (K operands of phase 1, then
  // V operands of phase 2), stream through one ring read AHEAD operands
  // ahead; operand u of a step of parity par sits in slot (u + NOPS par) % RING
  // (steps alternate parity, so every slot index is a compile-time constant).
  u32x4 op[RING];
  auto slot = [&](int par, int u) __attribute__((always_inline)) { return (u + NOPS * par) % RING; };
  auto read_op = [&](int par, int u, uint32_t ta, uint32_t tv) __attribute__((always_inline)) {
    if (u < NKOP)
      op[slot(par, u)] = kread(ta, u);
    else if (u < NOPS)
      op[slot(par, u)] = vread(tv, u - NKOP);
  };

  // S^T MFMA x (0..71) of a tile into acc: K operand u = x / 2, head tile
  // x % 2. With v_ops, the read-ahead runs on into the V operands of tv.
  auto s_mfma = [&](f32x4 (&acc)[2][2], int par, uint32_t ta, uint32_t tv, bool v_ops, int x)
                    __attribute__((always_inline)) {
    const int u = x >> 1, ht = x & 1, kt = u & 1, ks = u >> 1;
    if (ht == 0 && (u + AHEAD < NKOP || v_ops)) read_op(par, u + AHEAD, ta, tv);
    if (ks == 0)
      Mm::v0(acc[kt][ht], op[slot(par, u)], qop[ht][0]);
    else
      Mm::v(acc[kt][ht], op[slot(par, u)], qop[ht][ks]);
  };
  // S^T of the first tile (the prologue, parity of step -1).
  auto s_chain = [&](f32x4 (&acc)[2][2], uint32_t ta) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) read_op(1, u, ta, 0);
#pragma unroll
    for (int x = 0; x < 2 * NKOP; ++x) s_mfma(acc, 1, ta, 0, false, x);
  };

  // Rescale of the O^T tiles of head tile ht, each lane by its head's alpha,
  // when one of the tile's 16 row maxima grew (rescale_ht[ht]): with the
  // exact running max every growth rescales, and nothing else does. The empty
  // asm statements keep one tile's reads, multiplies and writes together
  // (unfenced, the compiler would hold all products in VGPRs at once). The
  // next MFMA reading these tiles is in phase 2, many instructions later, past
  // the wait states a VALU write needs before an MFMA reads it.
  bool rescale_ht[2] = {false, false};
  auto rescale_tiles = [&](int ht) __attribute__((always_inline)) {
    if (rescale_ht[ht]) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        asm volatile("" : "+a"(oacc[dt][ht]));
        oacc[dt][ht] *= alpha[ht];
        asm volatile("" : "+a"(oacc[dt][ht]));
      }
    }
  };

  // End of step j: this wave's copies of tile j+3 have landed (with V read
  // out of the K rows; else its copies of V_{j+1} and K_{j+2}), barrier, then
  // the copies into the slots step j left. Tile j+3 is waited for one step
  // early so that it is visible during step j+1, whose last MFMAs read the
  // first K operands of step j+2 from it (see step()).
  auto end_step = [&](int j) __attribute__((always_inline)) {
    if (VALIAS) {
      wait_copies_below(0);
      barrier_keep_copies();
      if (j + 4 < n_tiles) issue_k(j + 4);
    } else {
      wait_vmem();
      barrier_keep_copies();
      if (j + 3 < n_tiles) issue_k(j + 3);
      if (j + 2 < n_tiles) issue_v(j + 2);
    }
  };
  auto next_k_copy = [&](int j) __attribute__((always_inline)) { return VALIAS ? j + 4 : j + 3; };

  // Step j: softmax of tile j (scores sb), S^T of tile j+1 into sa, O^T +=
  // V_j^T P_j^T. On the last step the S^T of the (absent) next tile reads a
  // stale ring slot and is discarded.
  auto step = [&](int j, f32x4 (&sb)[2][2], f32x4 (&sa)[2][2], int par) __attribute__((always_inline)) {
    const uint32_t ta = ktile(j + 1);
    const uint32_t tv = vtile(j);
    const uint32_t tn = ktile(j + 2);
    // The first AHEAD operands of this step were read at the end of the step
    // before (with V read out of the K rows); else read them now.
    if (!VALIAS) {
#pragma unroll
      for (int u = 0; u < AHEAD; ++u) read_op(par, u, ta, tv);
    }
    // The scores were complete one MFMA phase ago; order the reads here.
    asm volatile("s_nop 0" : "+v"(sb[0][0]), "+v"(sb[0][1]), "+v"(sb[1][0]), "+v"(sb[1][1]));
    // Only the last list tile can be partial: keys past n_valid are masked.
    const int nk = n_valid - visit(j) * TB;
    if (nk < TB) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * kt + 4 * G + i >= nk) sb[kt][ht][i] = -INFINITY;
    }
    // Row max of each head (in-lane, then the 4 lanes of the head) and the
    // running-max update: exact, so any growth moves m.
    float m_new[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float mq = max3(sb[0][ht][0], sb[0][ht][1], sb[0][ht][2]);
      mq = max3(mq, sb[0][ht][3], sb[1][ht][0]);
      mq = max3(mq, sb[1][ht][1], sb[1][ht][2]);
      mq = fmaxf(mq, sb[1][ht][3]);
      const float mx = quad_max(mq) * p.scale_log2;
      const bool upd = mx > m_run[ht];
      m_new[ht] = upd ? mx : m_run[ht];  // finite: every tile has a valid key
      alpha[ht] = upd ? fast_exp2(m_run[ht] - m_new[ht]) : 1.f;
      m_run[ht] = m_new[ht];
      rescale_ht[ht] = j > 0 && __builtin_amdgcn_ballot_w64(upd) != 0;  // O is zero at j = 0
    }
    float rs[2] = {0.f, 0.f};
    // Phase 1: S^T(j+1); MFMAs 0 .. EXP_GAPS - 1 carry the exponentials
    // (one pair of scores each), then the rescale of O^T if a max grew.
    auto seg = [&](int x0, int x1) __attribute__((always_inline)) {
#pragma unroll
      for (int x = x0; x < x1; ++x) {
        s_mfma(sa, par, ta, tv, true, x);
        if (x < EXP_GAPS) {
          // head tile x % 2, scores e, e + 1 of it (e = 0, 2, 4, 6 over kt, i)
          const int ht = x & 1, e = 2 * (x >> 1);
          const int kt = e >> 2, i = e & 3;
          const float x0 = fast_exp2(__builtin_fmaf(sb[kt][ht][i], p.scale_log2, -m_new[ht]));
          const float x1 = fast_exp2(__builtin_fmaf(sb[kt][ht][i + 1], p.scale_log2, -m_new[ht]));
          pop[ht][e >> 1] = T::pack2(x0, x1);
          rs[ht] += x0 + x1;
          asm volatile("" ::"v"(pop[ht][e >> 1]), "v"(rs[ht]));
        }
      }
    };
    seg(0, EXP_GAPS);
    // Rare once the row maxima are met (see visit()): one branch, laid out of
    // line, keeps the common path free of taken jumps.
    if (__builtin_expect(rescale_ht[0] || rescale_ht[1], 0)) {
      rescale_tiles(0);
      rescale_tiles(1);
    }
    seg(EXP_GAPS, 2 * NKOP);
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) l_run[ht] = __builtin_fmaf(l_run[ht], alpha[ht], rs[ht]);
    // Phase 2: O^T += V^T P^T, MFMA q: d tile q / 2 (operand NKOP + q / 2),
    // head tile q % 2.
#pragma unroll
    for (int q = 0; q < 2 * NDT; ++q) {
      const int dt = q >> 1, ht = q & 1, u = NKOP + dt;
      if (ht == 0) {
        if (u + AHEAD < NOPS)
          read_op(par, u + AHEAD, ta, tv);
        else if (VALIAS)  // the next step's first K operands (K_{j+2}: landed at end_step(j-1))
          op[slot(par, u + AHEAD)] = kread(tn, u + AHEAD - NOPS);
      }
      Mm::a(oacc[dt][ht], op[slot(par, u)], pop[ht]);
      if (q == PREP_AT) prep_k(next_k_copy(j));
    }
    end_step(j);
  };

  // Prologue: the first tiles in flight, S^T of tile 0.
  if (n_tiles > 0) {
    if (VALIAS) {
      for (int i = 0; i < 3 && i < n_tiles; ++i) {
        prep_k(i);
        issue_k(i);
      }
      wait_copies_below((min(n_tiles, 3) - 1) * KCOPY);
    } else {
      prep_k(0);
      issue_k(0);
      if (n_tiles > 1) {
        prep_k(1);
        issue_k(1);
      }
      issue_v(0);
      wait_vmem();
    }
    barrier_keep_copies();
    s_chain(s0, ktile(0));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0[0][0]), "+v"(s0[0][1]), "+v"(s0[1][0]), "+v"(s0[1][1]));
    prep_k(next_k_copy(-1));
    end_step(-1);
    if (VALIAS) {
#pragma unroll
      for (int u = 0; u < AHEAD; ++u) read_op(0, u, ktile(1), vtile(0));
    }
  }
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, s0, s1, 0);
    if (j + 1 < n_tiles) step(j + 1, s1, s0, 1);
  }

  // Epilogue: O = acc / l, LSE = ln2 * (m + log2 l); no valid key -> 0 / -inf.
  // O goes through the ring (free once every copy has landed and every wave
  // has passed its last step): wave w writes its 32 heads x 512 as 32 rows
  // of 1 KB with the 16-byte chunks of row r XOR-swizzled by r (conflict-free
  // on both sides), then stores one whole head row per instruction.
#pragma unroll
  for (int dt = 0; dt < NDT; dt += 2)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(oacc[dt][0]), "+a"(oacc[dt][1]), "+a"(oacc[dt + 1][0]), "+a"(oacc[dt + 1][1]));
  wait_vmem();
  __syncthreads();
  static_assert(NWAVE * 32 * DV * 2 <= L_BASE, "O staging fits in the ring");
  char* const stage = (char*)s_mem + w * (32 * DV * 2);
  auto st_at = [&](int r, int ch) __attribute__((always_inline)) { return stage + r * (DV * 2) + ((ch ^ (r & 63)) << 4); };
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const float lt = quad_sum(l_run[ht]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r = 16 * ht + n;
    const bool head_ok = active && head0 + r < p.Hq;
    // With o_lo, the fp32 residual O - rounded(O) goes to HBM straight from
    // the registers (4 consecutive columns per lane and store).
    float* const olo = (p.o_lo && head_ok) ? p.o_lo + (int64_t)t * p.ol_st + (int64_t)(head0 + r) * p.ol_sh : nullptr;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float x0 = oacc[dt][ht][0] * inv, x1 = oacc[dt][ht][1] * inv;
      const float x2 = oacc[dt][ht][2] * inv, x3 = oacc[dt][ht][3] * inv;
      u32x2 v;
      v[0] = T::pack2(x0, x1);
      v[1] = T::pack2(x2, x3);
      // columns 16 dt + 4 G .. +3: chunk 2 dt + G / 2, bytes 8 (G % 2) in it
      *(u32x2*)(st_at(r, 2 * dt + (G >> 1)) + 8 * (G & 1)) = v;
      if (olo) {
        const f32x2 r0 = T::unpack2(v[0]), r1 = T::unpack2(v[1]);
        *(float4*)(olo + 16 * dt + 4 * G) = make_float4(x0 - r0[0], x1 - r0[1], x2 - r1[0], x3 - r1[1]);
      }
    }
    if (head_ok && G == 0)
      p.lse[(int64_t)t * p.Hq + head0 + r] = lt > 0.f ? (m_run[ht] + log2f(lt)) * kLn2 : -INFINITY;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (active) {
    uint16_t* const ob = (uint16_t*)p.o + (int64_t)t * p.o_st + (int64_t)head0 * p.o_sh;
    const int nh = min(32, p.Hq - head0);  // valid heads of this wave (a padded last tile)
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      const u32x4 v = *(const u32x4*)st_at(r, lane);
      if (r < nh) *(u32x4*)(ob + (int64_t)r * p.o_sh + 8 * lane) = v;
    }
  }
}

}  // namespace
}  // namespace fa

// Kernel entry points (names are looked up by the library at run time):
// fa_topk16_<dtype>_v<1: V is the first 512 columns of K, 0: V of its own>.
#define FA_TOPK16_KERNEL(TN, T, VA)                                                                   \
  extern "C" __global__ void __launch_bounds__(256, 1) fa_topk16_##TN##_v##VA(const fa::TopkParams p) { \
    fa::topk16_body<fa::T, VA != 0>(p);                                                                 \
  }
FA_TOPK16_KERNEL(bf16, BF16, 1)
FA_TOPK16_KERNEL(bf16, BF16, 0)
FA_TOPK16_KERNEL(f16, F16, 1)
FA_TOPK16_KERNEL(f16, F16, 0)
