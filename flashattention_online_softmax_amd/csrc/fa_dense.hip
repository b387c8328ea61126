// Dense, causal, masked, GQA and block-sparse attention forward for gfx950.
//
// Method: the online-softmax forward of the "FlashAttention correctness
// verification" page (tiled computation and loop-invariant sections): for each
// KV tile, S = scale * Q K^T, m' = max(m, rowmax S), l' = l * e^(m - m') +
// rowsum e^(S - m'), O' = O * e^(m - m') + e^(S - m') V, finally O = O / l and
// LSE = m + ln l. The max is exact (every growth rescales), as the sparse-MLA
// page of flash-attention prescribes for the exact-max forward.
//
// Work decomposition (MI355X): one workgroup of NW waves owns MPH consecutive
// query rows of HP query heads that share one KV head (HP > 1 packs GQA heads
// so that a single K/V tile in LDS serves them all). Every wave owns QT tiles
// of 32 query rows. With 8 waves of 32 rows a wave needs < 256 registers, so
// two waves share each SIMD and one wave's softmax (VALU) overlaps the
// other's MFMA work. Workgroups are numbered so that the longest causal tiles
// start first and every KV head maps to one XCD (consecutive workgroup ids go
// to consecutive XCDs and the KV-head index is the fastest-varying part).
//
// Per 64-key tile:
//   * K and V tiles are copied HBM -> VGPR -> LDS, double buffered, one tile
//     ahead of the compute, with an XOR swizzle of the 16-byte chunks so that
//     the MFMA operand reads below hit distinct LDS banks.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T
//     resident in VGPRs as the B operand). In the result each lane owns one
//     query column and 16 keys of it, so the row max and row sum are in-lane
//     reductions plus a single v_permlane32_swap between the wave halves.
//   * p = exp2(s * scale*log2e - m) on v_exp_f32 (one FMA + one exp per
//     score), m being the running max already in the exp2 domain; l
//     accumulates the fp32 p; p is rounded to 16 bits.
//   * O^T += V^T P^T on MFMA: P^T is already in B-operand layout (each lane
//     owns its query), V^T is read from the row-major V tile with
//     ds_read_b64_tr_b16, whose key order is chosen to match the key order in
//     which the S^T accumulator holds P. The rescale by e^(m - m') is then a
//     per-lane scalar multiply.
// Epilogue: O = acc / l rounded to the output dtype, LSE = ln2 * (m + log2 l)
// in fp32 (m being the running max in the exp2 domain); rows with no key give
// O = 0 and LSE = -inf.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BN = 64;  // keys per tile (16-bit path)

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

struct Work {
  int b, hkv, hq, wg_row0, row0, Lq, Lk;
};

// Decodes blockIdx.x into (query block, head group, KV head, batch); the
// last query block comes first (longest causal rows first) and the KV-head
// index varies fastest, so all query heads of one KV head land on one XCD.
template <int NW, int QT, int HP>
__device__ __forceinline__ Work decode_work(const FwdParams& p) {
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * QT * 32;
  const int w = threadIdx.x >> 6;
  const int BHkv = p.B * p.Hkv;
  const int per_mb = BHkv * p.n_hgroups;
  const int id = blockIdx.x;
  const int mb_rank = id / per_mb;
  const int r = id - mb_rank * per_mb;
  const int mb = p.n_mblocks - 1 - mb_rank;
  const int hg = r / BHkv;
  const int bkv = r - hg * BHkv;
  Work wk;
  wk.b = bkv / p.Hkv;
  wk.hkv = bkv - wk.b * p.Hkv;
  const int hp = w / WPH, wi = w - (w / WPH) * WPH;
  wk.hq = wk.hkv * p.G + hg * HP + hp;
  wk.wg_row0 = mb * MPH;
  wk.row0 = wk.wg_row0 + wi * QT * 32;
  int lq = p.Sq, lk = p.Skv;
  if (p.seqlens_q) lq = max(0, min(p.seqlens_q[wk.b], p.Sq));
  if (p.seqlens_k) lk = max(0, min(p.seqlens_k[wk.b], p.Skv));
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

// Number of 64-key tiles of a dense (optionally causal) workgroup.
template <bool CAUSAL>
__device__ __forceinline__ int dense_tiles(const Work& wk, int mph, int bn) {
  if (wk.wg_row0 >= wk.Lq) return 0;
  int kend = wk.Lk;
  if (CAUSAL) {
    const int last_row = min(wk.wg_row0 + mph, wk.Lq) - 1;
    kend = min(kend, last_row + (wk.Lk - wk.Lq) + 1);
  }
  return kend > 0 ? (kend + bn - 1) / bn : 0;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (fp16 / bf16), D in {64, 128}.
// ---------------------------------------------------------------------------
template <class T, int D, int QT, int NW, int HP, bool CAUSAL, bool MASK, bool SPARSE>
__global__ void __launch_bounds__(NW * 64, NW / 4) fwd16_kernel(const FwdParams p) {
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * QT * 32;
  constexpr int DS = D / 16;  // MFMA k-steps over D for S^T
  constexpr int DT = D / 32;  // 32-wide d tiles of O^T
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int NT = NW * 64;
  constexpr int LOADS = BN * CH / NT;
  static_assert(BN * CH % NT == 0, "tile copy must divide evenly");
  static_assert(!SPARSE || MPH == 128, "block-sparse needs 128 query rows per head");

  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][BN * D];
  __shared__ int s_kstart[SPARSE ? 512 : 1];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;
  const Work wk = decode_work<NW, QT, HP>(p);
  const int diag = wk.Lk - wk.Lq;  // key j is visible to row i iff j <= i + diag

  int n_iter;
  if (SPARSE)
    n_iter = build_sparse_tiles(p, wk, wk.wg_row0 / 128, s_kstart, &s_n);
  else
    n_iter = dense_tiles<CAUSAL>(wk, MPH, BN);

  const uint16_t* qg = (const uint16_t*)p.q + wk.b * p.q_sb + wk.hq * p.q_sh;
  const uint16_t* kg = (const uint16_t*)p.k + wk.b * p.k_sb + wk.hkv * p.k_sh;
  const uint16_t* vg = (const uint16_t*)p.v + wk.b * p.v_sb + wk.hkv * p.v_sh;

  // Q^T operands (B operand of S^T = K Q^T): lane holds Q[row][16 ds + 8 h .. +7].
  u32x4 qop[QT][DS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int row = wk.row0 + 32 * t + c;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (row < p.Sq) z = *(const u32x4*)(qg + (int64_t)row * p.q_ss + 16 * ds + 8 * h);
      qop[t][ds] = z;
    }
  }

  f32x16 oacc[QT][DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[t][dt][i] = 0.f;
  }

  // K/V tile staging: thread copies LOADS 16-byte chunks of each tile.
  u32x4 kreg[LOADS], vreg[LOADS];
  auto tile_start = [&](int it) { return SPARSE ? s_kstart[it] : it * BN; };
  auto gload = [&](int kstart) {
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int idx = tid + n * NT;
      const int row = idx / CH, ch = idx % CH;
      const int key = kstart + row;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key < wk.Lk) {
        zk = *(const u32x4*)(kg + (int64_t)key * p.k_ss + ch * 8);
        zv = *(const u32x4*)(vg + (int64_t)key * p.v_ss + ch * 8);
      }
      kreg[n] = zk;
      vreg[n] = zv;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int idx = tid + n * NT;
      const int row = idx / CH, ch = idx % CH;
      *(u32x4*)&s_k[buf][row * D + ((ch ^ kswz<D>(row)) << 3)] = kreg[n];
      *(u32x4*)&s_v[buf][row * D + ((ch ^ vswz<D>(row)) << 3)] = vreg[n];
    }
  };

  if (n_iter > 0) {
    gload(tile_start(0));
    lstore(0);
    if (n_iter > 1) gload(tile_start(1));
  }
  __syncthreads();

  // Mask rows of this lane's queries (only dereferenced for rows < Sq).
  const uint8_t* mrow[QT];
  if (MASK) {
#pragma unroll
    for (int t = 0; t < QT; ++t)
      mrow[t] = p.mask + wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)(wk.row0 + 32 * t + c) * p.m_ss;
  }

  // tr-read geometry of the V operand (see lds_read_tr16): lane reads row
  // vrow (+8 for keys 8..15 of a 16-key step) at column vcol of a d tile.
  const int vrow = 4 * h + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int kstart = tile_start(it);
    const uint16_t* sk = s_k[buf];
    const uint16_t* sv = s_v[buf];

    // A wave whose rows all lie past Lq, or whose last row cannot see this
    // tile (causal), has nothing to add: it only helps with the tile copies.
    const bool active = wk.row0 < wk.Lq && !(CAUSAL && kstart > wk.row0 + QT * 32 - 1 + diag);
    if (active) {
    // Mask bytes for this tile: 4 consecutive keys per (t, kt, g).
    uint32_t mbits[QT][2][4];
    if (MASK) {
      const bool vec = p.mask_vec4 && (kstart + BN <= p.Skv);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const bool rv = (wk.row0 + 32 * t + c) < p.Sq;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int key0 = kstart + kt * 32 + 8 * g + 4 * h;
            uint32_t bits = 0x01010101u;
            if (rv) {
              if (vec) {
                bits = *(const uint32_t*)(mrow[t] + key0);
              } else {
                bits = 0;
                for (int e = 0; e < 4; ++e)
                  bits |= (uint32_t)((key0 + e < p.Skv) ? mrow[t][key0 + e] : 1) << (8 * e);
              }
            }
            mbits[t][kt][g] = bits;
          }
      }
    }

    // S^T = K Q^T
    f32x16 s[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kt][t][i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = kt * 32 + c;
        const u32x4 kop = *(const u32x4*)&sk[row * D + (((2 * ds + h) ^ kswz<D>(row)) << 3)];
#pragma unroll
        for (int t = 0; t < QT; ++t) s[kt][t] = T::mfma(kop, qop[t][ds], s[kt][t]);
      }
    }

    // Masking: only tiles that touch a boundary, the diagonal or a mask.
    const bool edge = (kstart + BN > wk.Lk) || (wk.row0 + QT * 32 > wk.Lq) ||
                      (CAUSAL && kstart + BN - 1 > wk.row0 + diag);
    if (MASK || edge) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int qrow = wk.row0 + 32 * t + c;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kstart + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            bool ok = key < wk.Lk && qrow < wk.Lq;
            if (CAUSAL) ok = ok && key <= qrow + diag;
            if (MASK) ok = ok && ((mbits[t][kt][i >> 2] >> (8 * (i & 3))) & 0xffu) == 0u;
            if (!ok) s[kt][t][i] = -INFINITY;
          }
      }
    }

    // Online softmax (exact running max) and P packing.
    u32x4 pop[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][t][i]);
      mx = half_max(mx);
      // The running max is kept in the exp2 domain (m = round(max s * c)), so
      // that alpha is exactly 1 when the max does not move.
      const float m_new = fmaxf(m_run[t], mx * p.scale_log2);
      const float mc = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[t] - mc);
      m_run[t] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(__builtin_fmaf(s[kt][t][i], p.scale_log2, -mc));
          s[kt][t][i] = e;
          rs += e;
        }
      l_run[t] = l_run[t] * alpha + rs;
      // alpha is exactly 1 for a row whose max did not move: skip the
      // rescale when that holds for every row of the wave.
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[t][dt][i] *= alpha;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, j = ks & 1;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = T::pack2(s[kt][t][8 * j + 2 * e], s[kt][t][8 * j + 2 * e + 1]);
        pop[t][ks] = v;
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r0 = (ks >> 1) * 32 + (ks & 1) * 16 + vrow;
      const int r1 = r0 + 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = 32 * dt + vcol;
        const int ch = col >> 3, off = col & 7;
        const u32x2 lo = lds_read_tr16(&sv[r0 * D + ((ch ^ vswz<D>(r0)) << 3) + off]);
        const u32x2 hi = lds_read_tr16(&sv[r1 * D + ((ch ^ vswz<D>(r1)) << 3) + off]);
        const u32x4 vop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int t = 0; t < QT; ++t) oacc[t][dt] = T::mfma(vop, pop[t][ks], oacc[t][dt]);
      }
    }
    }  // active

    if (it + 1 < n_iter) lstore(buf ^ 1);
    if (it + 2 < n_iter) gload(tile_start(it + 2));
    __syncthreads();
  }

  // Epilogue.
  uint16_t* og = (uint16_t*)p.o + wk.b * p.o_sb + wk.hq * p.o_sh;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float lt = half_sum(l_run[t]);
    const int qrow = wk.row0 + 32 * t + c;
    if (qrow < p.Sq) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = og + (int64_t)qrow * p.o_ss;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v;
          v[0] = T::pack2(oacc[t][dt][4 * g] * inv, oacc[t][dt][4 * g + 1] * inv);
          v[1] = T::pack2(oacc[t][dt][4 * g + 2] * inv, oacc[t][dt][4 * g + 3] * inv);
          *(u32x2*)(orow + 32 * dt + 8 * g + 4 * h) = v;
        }
      if (h == 0)
        p.lse[((int64_t)wk.b * p.Hq + wk.hq) * p.Sq + qrow] =
            lt > 0.f ? (m_run[t] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

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
    n_iter = dense_tiles<CAUSAL>(wk, MPH, BN32);
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
    mx = half_max(mx);
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new;
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

template <class T, int D, bool CAUSAL, bool MASK>
hipError_t launch16_dense(FwdParams& p, hipStream_t st) {
  constexpr int NW = 8, QT = 1, HP = 1;
  dim3 grid;
  set_grid<NW, QT, HP>(p, grid);
  hipLaunchKernelGGL((fwd16_kernel<T, D, QT, NW, HP, CAUSAL, MASK, false>), grid, dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch16_sparse(FwdParams& p, hipStream_t st) {
  // 128 query rows per head (one query block); with an even GQA group two
  // heads of the group share each K/V tile.
  dim3 grid;
  if (p.G % 2 == 0) {
    set_grid<8, 1, 2>(p, grid);
    hipLaunchKernelGGL((fwd16_kernel<T, D, 1, 8, 2, false, false, true>), grid, dim3(512), 0, st, p);
  } else {
    set_grid<4, 1, 1>(p, grid);
    hipLaunchKernelGGL((fwd16_kernel<T, D, 1, 4, 1, false, false, true>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK, bool SPARSE>
hipError_t launch32(FwdParams& p, hipStream_t st) {
  dim3 grid;
  set_grid<4, 1, 1>(p, grid);
  hipLaunchKernelGGL((fwd32_kernel<D, 1, CAUSAL, MASK, SPARSE>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch16(bool causal, bool has_mask, bool sparse, FwdParams& p, hipStream_t st) {
  if (sparse) return launch16_sparse<T, D>(p, st);
  if (causal) return has_mask ? launch16_dense<T, D, true, true>(p, st) : launch16_dense<T, D, true, false>(p, st);
  return has_mask ? launch16_dense<T, D, false, true>(p, st) : launch16_dense<T, D, false, false>(p, st);
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
  if (dt == Dt::F16) return D == 128 ? launch16<F16, 128>(causal, has_mask, sparse, p, stream)
                                     : launch16<F16, 64>(causal, has_mask, sparse, p, stream);
  return D == 128 ? launch16<BF16, 128>(causal, has_mask, sparse, p, stream)
                  : launch16<BF16, 64>(causal, has_mask, sparse, p, stream);
}

}  // namespace fa
