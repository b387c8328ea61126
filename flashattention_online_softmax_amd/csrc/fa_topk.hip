// Top-k gathered sparse MLA forward for gfx950 (one shared KV head).
//
// Method: per token t, attention of every query head over the keys named in
// idx[t, :] (the sparse-MLA forward of the flash-attention SM100 page,
// background section), with the exact running max of that page (threshold
// 0: any growth of the row max rescales O and l, so the largest p of a row
// is exactly 1.0 before it is rounded for P.V). The online-softmax
// recurrence is the one of the "FlashAttention correctness verification"
// page (tiled computation / loop invariant).
//
// Decomposition (MI355X): one workgroup of 4 waves per (token, 128-head
// tile); wave w owns 32 heads. Its Q^T (32 heads x 576) stays in VGPRs as
// the B operand of S^T = K_g Q^T; its O^T accumulator (512 x 32 fp32) lives
// in the accumulation registers. The gathered key rows (1152 bytes each) are
// copied straight from HBM/L2 into LDS with global_load_lds_dwordx4 (no VGPR
// staging), 32 rows per tile, double buffered in two distinct LDS arrays so
// that the copy of tile i+1 overlaps the MFMA work on tile i. When V is the
// first 512 columns of K (the MLA latent), P.V reads V straight out of the
// gathered K rows; otherwise V rows are gathered the same way.
//
// The valid entries of idx[t, :] are first compacted into LDS (list order
// kept, negative slots dropped), so only the last tile of a token can be
// partial; its padding rows point at a valid key and are masked to -inf.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int DQK = 576, DV = 512;
constexpr int TBN = 32;              // gathered keys per tile
constexpr int CHK = DQK / 8;         // 16-byte chunks per K row (72)
constexpr int CHV = DV / 8;          // 16-byte chunks per V row (64)
constexpr int KDMA_W = TBN * CHK / 64 / 4;  // LDS-DMA instructions per wave per K tile (9)
constexpr int VDMA_W = TBN * CHV / 64 / 4;  // ... per V tile (8)
constexpr int WMAX = 4096;           // longest index row held in LDS

// Swizzle of the 16-byte chunk index inside aligned groups of 8 (K rows are
// 1152 bytes, so consecutive rows alternate between the two halves of the 64
// LDS banks; x(row) is a bijection of row/2 onto 0..7 whose bit 2 differs
// between rows 4a and 4a + 2).
__device__ __forceinline__ int kx(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int kphys(int lc, int row) { return (lc & ~7) | ((lc & 7) ^ kx(row)); }
// V rows (separate V tensor) are 1024 bytes: 4-chunk groups XOR 4*(row%4).
__device__ __forceinline__ int vphys(int lc, int row) { return lc ^ ((row & 3) << 2); }

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <class T, bool VALIAS>
struct TopkCtx {
  const TopkParams& p;
  const int* s_list;
  int n_valid;
  int w, lane, h, c;
  bool active;

  // Issue the LDS-DMA gather of tile `it` into (sk, sv).
  __device__ __forceinline__ void issue(int it, uint16_t* sk, uint16_t* sv) const {
    const uint16_t* kg = (const uint16_t*)p.k;
    const int base = it * TBN;
#pragma unroll
    for (int j = 0; j < KDMA_W; ++j) {
      const int P = (w * KDMA_W + j) * 64 + lane;  // chunk position in the tile
      const int row = P / CHK, ph = P - (P / CHK) * CHK;
      const int slot = base + row;
      const int key = s_list[slot < n_valid ? slot : 0];
      const int lc = kphys(ph, row);  // involution: logical chunk stored at ph
      const uint16_t* g = kg + (int64_t)key * p.k_ss + lc * 8;
      __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(sk + (w * KDMA_W + j) * 512), 16, 0, 0);
    }
    if (!VALIAS) {
      const uint16_t* vg = (const uint16_t*)p.v;
#pragma unroll
      for (int j = 0; j < VDMA_W; ++j) {
        const int P = (w * VDMA_W + j) * 64 + lane;
        const int row = P / CHV, ph = P % CHV;
        const int slot = base + row;
        const int key = s_list[slot < n_valid ? slot : 0];
        const uint16_t* g = vg + (int64_t)key * p.v_ss + vphys(ph, row) * 8;
        __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(sv + (w * VDMA_W + j) * 512), 16, 0, 0);
      }
    }
  }

  // One tile of online softmax + P.V for this wave's 32 heads.
  __device__ __forceinline__ void compute(int it, const uint16_t* sk, const uint16_t* sv,
                                          const u32x4 (&qop)[DQK / 16], f32x16 (&oacc)[DV / 32],
                                          float& m_run, float& l_run) const {
    if (!active) return;
    // S^T = K_g Q^T: 32 keys x 32 heads, 36 k-steps of 16.
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    const uint16_t* krow = sk + c * DQK;
#pragma unroll
    for (int ds = 0; ds < DQK / 16; ++ds) {
      const u32x4 kop = *(const u32x4*)(krow + kphys(2 * ds + h, c) * 8);
      s = T::mfma(kop, qop[ds], s);
    }
    const int nk = n_valid - it * TBN;  // valid keys in this tile (>= 1)
    if (nk < TBN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * h + (i & 3);
        if (r >= nk) s[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = half_max(mx);
    // running max in the exp2 domain: alpha is exactly 1 when it does not move
    const float m_new = fmaxf(m_run, mx * p.scale_log2);  // finite: every tile has a valid key
    const float mc = m_new;
    const float alpha = fast_exp2(m_run - mc);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -mc));
      s[i] = e;
      rs += e;
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    u32x4 pop[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) pop[j][e] = T::pack2(s[8 * j + 2 * e], s[8 * j + 2 * e + 1]);

    // O^T += V^T P^T, V^T read with ds_read_b64_tr_b16 in P's key order.
    const int vrow = 4 * h + ((lane & 15) >> 2);
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r0 = 16 * j + vrow, r1 = r0 + 8;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt) {
        const int col = 32 * dt + vcol;
        const int lc = col >> 3, off = col & 7;
        u32x2 lo, hi;
        if (VALIAS) {
          lo = lds_read_tr16(sk + r0 * DQK + kphys(lc, r0) * 8 + off);
          hi = lds_read_tr16(sk + r1 * DQK + kphys(lc, r1) * 8 + off);
        } else {
          lo = lds_read_tr16(sv + r0 * DV + vphys(lc, r0) * 8 + off);
          hi = lds_read_tr16(sv + r1 * DV + vphys(lc, r1) * 8 + off);
        }
        const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = T::mfma(vop, pop[j], oacc[dt]);
      }
    }
  }
};

template <class T, bool VALIAS>
__global__ void __launch_bounds__(256) topk_kernel(const TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[TBN * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[TBN * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[VALIAS ? 8 : TBN * DV];
  __shared__ __attribute__((aligned(16))) uint16_t s_v1[VALIAS ? 8 : TBN * DV];
  __shared__ int s_list[WMAX];
  __shared__ int s_wcount[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int t = blockIdx.x / p.n_htiles;
  const int ht = blockIdx.x - t * p.n_htiles;
  const int head = ht * 128 + w * 32 + c;
  const bool active = ht * 128 + w * 32 < p.Hq;

  // Compact the valid indices of row t into s_list (list order kept):
  // thread tid owns the slots [tid*spt, tid*spt + spt).
  const int32_t* irow = p.idx + (int64_t)t * p.idx_st;
  const int spt = (p.W + 255) / 256;
  int cnt = 0;
  for (int e = 0; e < spt; ++e) {
    const int s = tid * spt + e;
    if (s < p.W && irow[s] >= 0) ++cnt;
  }
  // exclusive scan of cnt over the workgroup
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wcount[w] = incl;
  __syncthreads();
  int off = incl - cnt;
  for (int ww = 0; ww < w; ++ww) off += s_wcount[ww];
  const int n_valid = s_wcount[0] + s_wcount[1] + s_wcount[2] + s_wcount[3];
  for (int e = 0; e < spt; ++e) {
    const int s = tid * spt + e;
    if (s < p.W) {
      const int x = irow[s];
      if (x >= 0) s_list[off++] = x;
    }
  }
  __syncthreads();

  // Q^T operands: lane holds Q[t, head, 16 ds + 8 h .. +7].
  u32x4 qop[DQK / 16];
  const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)t * p.q_st + (int64_t)head * p.q_sh;
#pragma unroll
  for (int ds = 0; ds < DQK / 16; ++ds) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (active) z = *(const u32x4*)(qrow + 16 * ds + 8 * h);
    qop[ds] = z;
  }
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  TopkCtx<T, VALIAS> cx{p, s_list, n_valid, w, lane, h, c, active};
  const int n_tiles = (n_valid + TBN - 1) / TBN;
  if (n_tiles > 0) cx.issue(0, s_k0, s_v0);
  for (int it = 0; it < n_tiles; it += 2) {
    // tile it lives in buffer 0, tile it + 1 in buffer 1
    wait_vmcnt0();
    __syncthreads();
    if (it + 1 < n_tiles) cx.issue(it + 1, s_k1, s_v1);
    cx.compute(it, s_k0, s_v0, qop, oacc, m_run, l_run);
    if (it + 1 < n_tiles) {
      wait_vmcnt0();
      __syncthreads();
      if (it + 2 < n_tiles) cx.issue(it + 2, s_k0, s_v0);
      cx.compute(it + 1, s_k1, s_v1, qop, oacc, m_run, l_run);
    }
  }

  // Epilogue: O = acc / l, LSE = ln2 * (m + log2 l); no valid key -> 0 / -inf.
  const float lt = half_sum(l_run);
  if (active) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = (uint16_t*)p.o + (int64_t)t * p.o_st + (int64_t)head * p.o_sh;
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v[0] = T::pack2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
        v[1] = T::pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * g + 4 * h) = v;
      }
    if (h == 0) p.lse[(int64_t)t * p.Hq + head] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <class T>
hipError_t launch_topk_t(TopkParams& p, hipStream_t st) {
  p.n_htiles = (p.Hq + 127) / 128;
  const dim3 grid((unsigned)(p.T * p.n_htiles));
  const bool alias = p.v == p.k && p.v_ss == p.k_ss;
  if (alias)
    hipLaunchKernelGGL((topk_kernel<T, true>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((topk_kernel<T, false>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(Dt dt, TopkParams& p, hipStream_t stream) {
  return dt == Dt::F16 ? launch_topk_t<F16>(p, stream) : launch_topk_t<BF16>(p, stream);
}

}  // namespace fa
