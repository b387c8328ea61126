// Attention forward launchers and the fp32 kernel for gfx950.
//
// Method: the online-softmax forward of the "FlashAttention correctness
// verification" page (tiled computation and loop-invariant sections): for each
// KV tile, S = scale * Q K^T, m' = max(m, rowmax S), l' = l * e^(m - m') +
// rowsum e^(S - m'), O' = O * e^(m - m') + e^(S - m') V, finally O = O / l and
// LSE = m + ln l. The reference max moves only when a tile's max exceeds it by
// more than the rescale threshold (the threshold branch of the flash-attention
// sparse-MLA exact-running-max guide); threshold 0 is the exact running max.
//
// This file holds
//   * fwd32_kernel: the fp32 path (v_mfma_f32_32x32x2f32, P kept in fp32,
//     32-key tiles staged in LDS as padded fp32 rows, one wave per 32 query
//     rows), D in {64, 128}; it exists for exactness, not speed;
//   * the launchers of the 16-bit kernels of fa_fwd16.hip, which live in the
//     separately compiled code object (fa_module.hip looks them up by name):
//     grid sizing for the dense, causal, masked, GQA and block-sparse modes,
//     for packed sequences (cu_seqlens) and for split-KV key ranges, whose
//     partial results the merge kernel of fa_split.hip combines.
// The work decomposition (rows per workgroup, XCD-aware order) is decode_work
// in fa_tiles.h, shared by every forward kernel.
#include <cstdio>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32, P kept in fp32), D in {64, 128}.
// One wave per 32 query rows, 32-key tiles. This path favours exactness over
// speed: K and V tiles are staged in LDS as fp32 rows.
// ---------------------------------------------------------------------------
template <int D, int HP, bool CAUSAL, bool MASK, bool SPARSE>
__global__ void __launch_bounds__(256) fwd32_kernel(const FwdParams p) {
  constexpr int NW = 4, QT = 1, BN32 = 32;
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * 32;
  constexpr int DT = D / 32;
  constexpr int KP = D + 1;  // padded K row (conflict-free column reads)
  static_assert(!SPARSE || MPH == 128, "block-sparse needs 128 query rows per head");

  __shared__ float s_k[BN32 * KP];
  __shared__ float s_v[BN32 * D];
  __shared__ int s_kstart[SPARSE ? 1536 : 1];
  __shared__ int s_n;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const Work wk = decode_work<NW, QT, HP>(p);
  const int diag = wk.Lk - wk.Lq;

  int n_iter;
  if (SPARSE) {
    // 128-key blocks -> four 32-key tiles each (tiles beyond Lk are skipped).
    const int n64 = build_sparse_tiles(p, wk, wk.wg_row0 / 128, s_kstart, &s_n);
    __syncthreads();
    if (tid == 0) {
      int n = 0;
      for (int i = 0; i < n64; ++i) {
        const int k0 = s_kstart[i];
        s_kstart[512 + n++] = k0;
        if (k0 + 32 < wk.Lk) s_kstart[512 + n++] = k0 + 32;
      }
      s_n = n;
    }
    __syncthreads();
    n_iter = s_n;
  } else {
    n_iter = dense_tiles<CAUSAL>(wk, MPH, BN32, diag);
  }

  const float* qg = (const float*)p.q + wk.b * p.q_sb + wk.hq * p.q_sh;
  const float* kg = (const float*)p.k + wk.b * p.k_sb + wk.hkv * p.k_sh;
  const float* vg = (const float*)p.v + wk.b * p.v_sb + wk.hkv * p.v_sh;
  const int qrow = wk.row0 + c;

  // Q^T operand: lane holds Q[qrow][2 ds + h].
  float qop[D / 2];
#pragma unroll
  for (int ds = 0; ds < D / 2; ++ds) qop[ds] = qrow < p.Sq ? qg[(int64_t)qrow * p.q_ss + 2 * ds + h] : 0.f;

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int it = 0; it < n_iter; ++it) {
    const int kstart = SPARSE ? s_kstart[512 + it] : it * BN32;
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < BN32 * D; idx += 256) {
      const int row = idx / D, col = idx % D;
      const int key = kstart + row;
      float kv = 0.f, vv = 0.f;
      if (key < wk.Lk) {
        kv = kg[(int64_t)key * p.k_ss + col];
        vv = vg[(int64_t)key * p.v_ss + col];
      }
      s_k[row * KP + col] = kv;
      s_v[row * D + col] = vv;
    }
    __syncthreads();

    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 2; ++ds)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(s_k[c * KP + 2 * ds + h], qop[ds], s, 0, 0, 0);

    const bool edge = (kstart + BN32 > wk.Lk) || (wk.row0 + 32 > wk.Lq) ||
                      (CAUSAL && kstart + BN32 - 1 > wk.row0 + diag);
    if (MASK || edge) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kstart + 8 * (i >> 2) + 4 * h + (i & 3);
        bool ok = key < wk.Lk && qrow < wk.Lq;
        if (CAUSAL) ok = ok && key <= qrow + diag;
        if (MASK && ok)
          ok = p.mask[wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)qrow * p.m_ss + key] == 0;
        if (!ok) s[i] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = half_max(mx) * p.scale_log2;
    // The reference max moves when the tile's max exceeds it by more than
    // the rescale threshold (0: exact running max).
    const bool upd = mx > m_run + p.rescale_thr;
    const float m_new = upd ? mx : m_run;
    const float mc = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = upd ? fast_exp2(m_run - mc) : 1.f;
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
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;

    // O^T += V^T P^T with k = 2 per MFMA: step i consumes p_i; lane half h
    // supplies key 8*(i/4) + 4*h + i%4.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * h + (i & 3);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(s_v[key * D + 32 * dt + c], s[i], oacc[dt], 0, 0, 0);
      }
  }

  const float lt = half_sum(l_run);
  if (qrow < p.Sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* orow = (float*)p.o + wk.b * p.o_sb + wk.hq * p.o_sh + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v = {oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                    oacc[dt][4 * g + 3] * inv};
        *(float4*)(orow + 32 * dt + 8 * g + 4 * h) = v;
      }
    if (h == 0)
      p.lse[((int64_t)wk.b * p.Hq + wk.hq) * p.Sq + qrow] =
          lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <int NW, int QT, int HP>
void set_grid(FwdParams& p, dim3& grid) {
  constexpr int MPH = (NW / HP) * QT * 32;
  p.n_mblocks = (p.Sq + MPH - 1) / MPH;
  p.n_hgroups = p.G / HP;
  grid = dim3((unsigned)p.n_mblocks * p.B * p.Hkv * p.n_hgroups);
}

// Launches kernel fa_fwd16_<tn>_d<D>_w<NW>_q<QT>_h<HP>_c<C>m<M>s<S>x<XM> of
// the 16-bit code object (XM: 0 BNSD, 1 packed variable-length, 2 split-KV
// partials, one workgroup per key range as well).
template <int NW, int QT, int HP>
hipError_t launch16_named(const char* tn, int D, bool causal, int mask, bool sparse, FwdParams& p,
                          hipStream_t st, int xm = 0) {
  dim3 grid;
  set_grid<NW, QT, HP>(p, grid);
  if (xm == 2) grid.x *= (unsigned)p.n_splits;
  char name[96];
  snprintf(name, sizeof(name), "fa_fwd16_%s_d%d_w%d_q%d_h%d_c%dm%ds%dx%d", tn, D, NW, QT, HP,
           causal ? 1 : 0, mask, sparse ? 1 : 0, xm);
  hipFunction_t fn = nullptr;
  hipError_t e = code_object_function(name, &fn);
  if (e != hipSuccess) return e;
  void* args[] = {&p};
  return hipModuleLaunchKernel(fn, grid.x, grid.y, grid.z, NW * 64, 1, 1, 0, st, args, nullptr);
}

hipError_t launch16(const char* tn, int D, bool causal, bool has_mask, bool sparse, FwdParams& p,
                    hipStream_t st) {
  // Dense: 8 waves of 32 query rows (256 rows per workgroup, two waves per
  // SIMD). A boolean mask whose rows are 16-byte chunks is staged through
  // LDS (mode 2), any other is loaded into registers (mode 1).
  if (!sparse) return launch16_named<8, 1, 1>(tn, D, causal, has_mask ? (p.mask_lds ? 2 : 1) : 0, false, p, st);
  // Block-sparse: 128 query rows per head (one query block); with an even
  // GQA group two heads of the group share each K/V tile.
  if (p.G % 2 == 0) return launch16_named<8, 1, 2>(tn, D, false, 0, true, p, st);
  return launch16_named<4, 1, 1>(tn, D, false, 0, true, p, st);
}

template <int D, bool CAUSAL, bool MASK, bool SPARSE>
hipError_t launch32(FwdParams& p, hipStream_t st) {
  dim3 grid;
  set_grid<4, 1, 1>(p, grid);
  hipLaunchKernelGGL((fwd32_kernel<D, 1, CAUSAL, MASK, SPARSE>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch32d(bool causal, bool has_mask, bool sparse, FwdParams& p, hipStream_t st) {
  if (sparse) return launch32<D, false, false, true>(p, st);
  if (causal) return has_mask ? launch32<D, true, true, false>(p, st) : launch32<D, true, false, false>(p, st);
  return has_mask ? launch32<D, false, true, false>(p, st) : launch32<D, false, false, false>(p, st);
}

}  // namespace

hipError_t launch_dense(Dt dt, int D, bool causal, bool has_mask, bool sparse, FwdParams& p,
                        hipStream_t stream) {
  if (dt == Dt::F32) return D == 128 ? launch32d<128>(causal, has_mask, sparse, p, stream)
                                     : launch32d<64>(causal, has_mask, sparse, p, stream);
  return launch16(dt == Dt::F16 ? "f16" : "bf16", D, causal, has_mask, sparse, p, stream);
}

hipError_t launch_varlen(Dt dt, int D, bool causal, FwdParams& p, hipStream_t stream) {
  return launch16_named<8, 1, 1>(dt == Dt::F16 ? "f16" : "bf16", D, causal, 0, false, p, stream, 1);
}

hipError_t launch_splitkv(Dt dt, int D, bool causal, FwdParams& p, hipStream_t stream) {
  hipError_t e = launch16_named<8, 1, 1>(dt == Dt::F16 ? "f16" : "bf16", D, causal, 0, false, p, stream, 2);
  if (e != hipSuccess) return e;
  MergeParams m;
  m.part_o = p.part_o;
  m.part_lse = p.part_lse;
  m.o = p.o;
  m.lse = p.lse;
  m.o_sb = p.o_sb;
  m.o_sh = p.o_sh;
  m.o_ss = p.o_ss;
  m.B = p.B;
  m.Hq = p.Hq;
  m.Sq = p.Sq;
  m.Dv = D;
  m.n_splits = p.n_splits;
  return launch_merge(dt, m, stream);
}

}  // namespace fa
