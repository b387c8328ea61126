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
// 16-bit kernel (fp16 / bf16), D in {64, 128}. One wave = 32 query rows.
// ---------------------------------------------------------------------------

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i fills LDS bytes [lds_addr + 16 i, +16).
// Issued through inline assembly so that the compiler does not hold later
// LDS reads of other buffers behind it; the kernel itself waits for these
// copies (s_waitcnt vmcnt) before the barrier that publishes their data.
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(gbase)
      : "memory", "m0");
}

// A pointer whose value is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits until at most N vector-memory operations of this wave are in flight
// (they retire in issue order for this counter).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not drain in-flight LDS copies (a full
// __syncthreads fence would). Each wave first waits for its own LDS
// operations; a wave that issued copies others read must wait for them
// itself before it reaches the barrier.
__device__ __forceinline__ void barrier_keep_copies() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copies of 64-key tiles (rows kstart .. kstart+63 of one K or V head) into
// LDS buffers of 64 rows x D elements stored with the 16-byte chunk swizzle.
// One copy instruction fills 64 consecutive chunks (1 KB) of LDS, lane i
// chunk 64n + i, so each lane fetches the logical chunk the swizzle keeps at
// that position (the XOR is an involution). The per-lane byte offset inside a
// tile is the same for every tile and is computed once. On the last, partial
// tile, rows at or past Lk fetch row Lk - 1 instead (finite data whose scores
// are masked), so nothing past the valid keys is ever read.
template <int D, int NW, bool IS_V>
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int NINST = BN * CH / 64;
  static constexpr int PER_WAVE = NINST / NW;
  static_assert(NINST % NW == 0, "tile copy must divide evenly over the waves");
  const char* g;      // head base
  int64_t row_bytes;  // row stride in bytes
  uint32_t off[PER_WAVE];

  __device__ __forceinline__ static int pos(int j) {
    return (((int)threadIdx.x >> 6) * PER_WAVE + j) * 64 + ((int)threadIdx.x & 63);
  }
  __device__ __forceinline__ static int chunk_row(int j) { return pos(j) / CH; }
  __device__ __forceinline__ static int chunk_col_bytes(int j) {
    const int row = pos(j) / CH, ph = pos(j) % CH;
    return (ph ^ (IS_V ? vswz<D>(row) : kswz<D>(row))) * 16;
  }

  // head is the same in every lane of the wave.
  __device__ __forceinline__ TileCopy(const uint16_t* head, int64_t row_stride)
      : g(uniform_ptr(head)), row_bytes(row_stride * 2) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) off[j] = (uint32_t)(chunk_row(j) * row_bytes + chunk_col_bytes(j));
  }

  // kstart, Lk and lds are the same in every lane of the wave.
  __device__ __forceinline__ void issue(int kstart, int Lk, const uint16_t* lds) const {
    kstart = __builtin_amdgcn_readfirstlane(kstart);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(
        lds_addr_of(lds) + (((int)threadIdx.x >> 6) * PER_WAVE) * 1024);
    const char* base = g + (int64_t)kstart * row_bytes;
    if (kstart + BN <= Lk) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) lds_copy16(base, off[j], l0 + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int r = min(chunk_row(j), Lk - 1 - kstart);
        lds_copy16(base, (uint32_t)(r * row_bytes + chunk_col_bytes(j)), l0 + j * 1024);
      }
    }
  }
};

// Two wave groups run one phase apart ("ping-pong"): per key tile j a wave
// has a VALU phase V(j) (mask, row max, rescale of O, exponentials, row sum,
// P packing) and an MFMA phase M(j) (scores of tile j+1 and O += P_j V_j).
// Group 0 runs M(-1) V(0) M(0) V(1) M(1) ..., group 1 the same one phase
// later, and every phase ends with a workgroup barrier, so on each SIMD one
// wave's softmax issues while the other wave's MFMAs run. Each SIMD holds
// one wave of each group (waves w and w + NW/2).
//
// K and V tiles live in three-deep LDS rings (tile t in slot t % 3). In
// global phase 2j+2 every wave copies K_{j+3} into the slot K_j used and
// V_{j+2} into the slot V_{j-1} used: both were last read in phase 2j+1 by
// group 1's M(j-1), before the barrier that closed it. The copies issued in
// a phase are waited for at the end of the next phase, well before their
// first reader (phase 2j+6).
template <class T, int D, int NW, int HP, bool CAUSAL, bool MASK, bool SPARSE>
__global__ void __launch_bounds__(NW * 64, NW / 4) fwd16_kernel(const FwdParams p) {
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * 32;
  constexpr int DS = D / 16;  // MFMA k-steps over D for S^T
  constexpr int DT = D / 32;  // 32-wide d tiles of O^T
  constexpr int TILE = BN * D;
  static_assert(!SPARSE || MPH == 128, "block-sparse needs 128 query rows per head");

  __shared__ __attribute__((aligned(16))) uint16_t s_kring[3 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t s_vring[3 * TILE];
  __shared__ int s_kstart[SPARSE ? 512 : 1];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;
  const int grp = w / (NW / 2);
  const Work wk = decode_work<NW, 1, HP>(p);
  const int diag = wk.Lk - wk.Lq;  // key j is visible to row i iff j <= i + diag
  const int qrow = wk.row0 + c;

  int n_iter;
  if (SPARSE)
    n_iter = build_sparse_tiles(p, wk, wk.wg_row0 / 128, s_kstart, &s_n);
  else
    n_iter = dense_tiles<CAUSAL>(wk, MPH, BN);
  // Tiles this wave works on: none if its rows are past Lq; under the causal
  // mask only the tiles that start at or before its last visible key.
  int n_act = n_iter;
  if (wk.row0 >= wk.Lq) {
    n_act = 0;
  } else if (CAUSAL && !SPARSE) {
    const int last_key = min(wk.row0 + 31, wk.Lq - 1) + diag;
    n_act = last_key < 0 ? 0 : min(n_iter, last_key / BN + 1);
  }

  const uint16_t* qg = (const uint16_t*)p.q + wk.b * p.q_sb + wk.hq * p.q_sh;
  const uint16_t* kg = (const uint16_t*)p.k + wk.b * p.k_sb + wk.hkv * p.k_sh;
  const uint16_t* vg = (const uint16_t*)p.v + wk.b * p.v_sb + wk.hkv * p.v_sh;

  // Q^T operands (B operand of S^T = K Q^T): lane holds Q[qrow][16 ds + 8 h .. +7].
  u32x4 qop[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    u32x4 z = {0u, 0u, 0u, 0u};
    if (qrow < p.Sq) z = *(const u32x4*)(qg + (int64_t)qrow * p.q_ss + 16 * ds + 8 * h);
    qop[ds] = z;
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 sc[2];  // scores of the tile the next V phase works on
  u32x4 pop[4];  // P of the tile the next M phase works on
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[kt][i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) pop[ks] = u32x4{0u, 0u, 0u, 0u};

  const uint8_t* mrow = nullptr;
  if (MASK) mrow = p.mask + wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)qrow * p.m_ss;
  auto tile_start = [&](int it) { return SPARSE ? s_kstart[it] : it * BN; };

  const TileCopy<D, NW, false> kcopy(kg, p.k_ss);
  const TileCopy<D, NW, true> vcopy(vg, p.v_ss);
  constexpr int NCOPY = TileCopy<D, NW, false>::PER_WAVE + TileCopy<D, NW, true>::PER_WAVE;

  // Per-lane element offsets of the MFMA operands inside a tile.
  // K (A operand of S^T): row kt*32 + c, logical chunk 2 ds + h.
  int koff[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = c * D + (((2 * ds + h) ^ kswz<D>(c)) << 3);
  // V (tr-read, see lds_read_tr16): rows vrow (+8) of each 16-key step,
  // column vcol of each d tile.
  const int vrow = 4 * h + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int col = 32 * dt + vcol;
    voff[dt] = vrow * D + (((col >> 3) ^ vswz<D>(vrow)) << 3) + (col & 7);
  }

  // M phase part 1: scores of a tile into sc (K operands read two MFMAs ahead).
  auto scores = [&](const uint16_t* kt_buf) {
    constexpr int NMF = 2 * DS;
    auto kread = [&](int i) -> u32x4 {
      return *(const u32x4*)&kt_buf[(i & 1) * 32 * D + koff[i >> 1]];
    };
    const f32x16 zero16 = {};
    u32x4 kq[3];
    kq[0] = kread(0);
    kq[1] = kread(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      if (i + 2 < NMF) kq[(i + 2) % 3] = kread(i + 2);
      sc[i & 1] = T::mfma(kq[i % 3], qop[i >> 1], i < 2 ? zero16 : sc[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // M phase part 2: O^T += V^T P^T (V operands read two MFMAs ahead).
  auto pv = [&](const uint16_t* vt_buf) {
    // One base address per d tile; the row offsets are immediates.
    const lds_u16* vb[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vb[dt] = lds_ptr(lds_addr_of(vt_buf) + 2 * voff[dt]);
    auto vread = [&](int m) -> u32x4 {
      const int dt = m >> 2, ks = m & 3;
      const int rb = ((ks >> 1) * 32 + (ks & 1) * 16) * D;  // vswz depends on row % 4 only
      const u32x2 lo = lds_read_tr16(vb[dt] + rb);
      const u32x2 hi = lds_read_tr16(vb[dt] + rb + 8 * D);
      const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
      return v;
    };
    u32x4 vq[3];
    vq[0] = vread(0);
    vq[1] = vread(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 4 * DT; ++m) {
      if (m + 2 < 4 * DT) vq[(m + 2) % 3] = vread(m + 2);
      oacc[m >> 2] = T::mfma(vq[m % 3], pop[m & 3], oacc[m >> 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: K_0, K_1, K_2, V_0, V_1 in flight.
  if (n_iter > 0) {
    kcopy.issue(tile_start(0), wk.Lk, s_kring);
    vcopy.issue(tile_start(0), wk.Lk, s_vring);
  }
  if (n_iter > 1) {
    kcopy.issue(tile_start(1), wk.Lk, s_kring + TILE);
    vcopy.issue(tile_start(1), wk.Lk, s_vring + TILE);
  }
  if (n_iter > 2) kcopy.issue(tile_start(2), wk.Lk, s_kring + 2 * TILE);
  // Make the compiler wait for the Q loads here, once: it does not see the
  // copies above, and otherwise would wait for its Q loads (vmcnt(0), which
  // drains copies in flight) at their first use inside the loop.
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) asm volatile("" ::"v"(qop[ds]));
  wait_vmem();
  __syncthreads();

  // Copies issued in global phase 2j+2: K_{j+3} into K_j's slot, V_{j+2}
  // into V_{j-1}'s slot. Returns whether this wave issued any.
  auto copies = [&](int j) {
    const bool ck = j + 3 < n_iter, cv = j + 2 < n_iter;
    if (ck) kcopy.issue(tile_start(j + 3), wk.Lk, s_kring + (j % 3) * TILE);
    if (cv) vcopy.issue(tile_start(j + 2), wk.Lk, s_vring + ((j + 2) % 3) * TILE);
    return ck || cv;
  };
  // End of a phase: this wave's copies issued one phase earlier are complete
  // (those of this phase may still fly), then the workgroup barrier.
  auto end_phase = [&](bool copied_now) {
    if (copied_now)
      wait_vmem_below<NCOPY>();
    else
      wait_vmem();
    barrier_keep_copies();
  };

  // V(j): mask, running max, rescale, exponentials, row sum, P packing.
  auto vphase = [&](int j) {
    const int kstart = tile_start(j);
    uint32_t mbits[2][4];
    if (MASK) {
      // 4 consecutive mask bytes per (kt, g).
      const bool vec = p.mask_vec4 && (kstart + BN <= p.Skv);
      const bool rv = qrow < p.Sq;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int key0 = kstart + kt * 32 + 8 * g + 4 * h;
          uint32_t bits = 0x01010101u;
          if (rv) {
            if (vec) {
              bits = *(const uint32_t*)(mrow + key0);
            } else {
              bits = 0;
              for (int e = 0; e < 4; ++e)
                bits |= (uint32_t)((key0 + e < p.Skv) ? mrow[key0 + e] : 1) << (8 * e);
            }
          }
          mbits[kt][g] = bits;
        }
    }
    const bool edge = (kstart + BN > wk.Lk) || (wk.row0 + 32 > wk.Lq) ||
                      (CAUSAL && kstart + BN - 1 > wk.row0 + diag);
    if (MASK || edge) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          bool ok = key < wk.Lk && qrow < wk.Lq;
          if (CAUSAL) ok = ok && key <= qrow + diag;
          if (MASK) ok = ok && ((mbits[kt][i >> 2] >> (8 * (i & 3))) & 0xffu) == 0u;
          if (!ok) sc[kt][i] = -INFINITY;
        }
    }
    // Exact running max kept in the exp2 domain (m = round(max s * c)), so
    // that alpha is exactly 1 when the max does not move. Two chains of
    // three-input maxima.
    float mq[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      mq[kt] = max3(sc[kt][0], sc[kt][1], sc[kt][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mq[kt] = max3(mq[kt], sc[kt][i], sc[kt][i + 1]);
      mq[kt] = fmaxf(mq[kt], sc[kt][15]);
    }
    const float mx = half_max(fmaxf(mq[0], mq[1]));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mc);
    m_run = m_new;
    // P rounded to the input type for the P V product; the row sum adds the
    // fp32 values.
    float rs[2] = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      const int kt = e >> 4, ii = e & 15;
      const float x0 = fast_exp2(__builtin_fmaf(sc[kt][ii], p.scale_log2, -mc));
      const float x1 = fast_exp2(__builtin_fmaf(sc[kt][ii + 1], p.scale_log2, -mc));
      pop[e >> 3][(e & 7) >> 1] = T::pack2(x0, x1);
      rs[(e >> 1) & 1] += x0 + x1;
    }
    l_run = __builtin_fmaf(l_run, alpha, rs[0] + rs[1]);
    // Rescale O only when some row's maximum moved (alpha is exactly 1
    // otherwise).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
  };

  // Group 1 starts one phase late.
  if (grp == 1) end_phase(false);
  // M(-1): scores of tile 0.
  if (n_act > 0) scores(s_kring);
  end_phase(false);
  for (int j = 0; j < n_iter; ++j) {
    // Group 0 runs V(j) in global phase 2j+1 and M(j) in 2j+2, group 1 in
    // 2j+2 and 2j+3; the copies belong to phase 2j+2.
    bool cp = false;
    if (grp == 1) cp = copies(j);
    if (j < n_act) vphase(j);
    end_phase(cp);
    cp = false;
    if (grp == 0) cp = copies(j);
    if (j < n_act) {
      if (j + 1 < n_act) scores(s_kring + ((j + 1) % 3) * TILE);
      pv(s_vring + (j % 3) * TILE);
    }
    end_phase(cp);
  }
  if (grp == 0) end_phase(false);

  // Epilogue.
  uint16_t* og = (uint16_t*)p.o + wk.b * p.o_sb + wk.hq * p.o_sh;
  const float lt = half_sum(l_run);
  if (qrow < p.Sq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = og + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v;
        v[0] = T::pack2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
        v[1] = T::pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(u32x2*)(orow + 32 * dt + 8 * g + 4 * h) = v;
      }
    if (h == 0)
      p.lse[((int64_t)wk.b * p.Hq + wk.hq) * p.Sq + qrow] =
          lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
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
  constexpr int NW = 8, HP = 1;
  dim3 grid;
  set_grid<NW, 1, HP>(p, grid);
  hipLaunchKernelGGL((fwd16_kernel<T, D, NW, HP, CAUSAL, MASK, false>), grid, dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch16_sparse(FwdParams& p, hipStream_t st) {
  // 128 query rows per head (one query block); with an even GQA group two
  // heads of the group share each K/V tile.
  dim3 grid;
  if (p.G % 2 == 0) {
    set_grid<8, 1, 2>(p, grid);
    hipLaunchKernelGGL((fwd16_kernel<T, D, 8, 2, false, false, true>), grid, dim3(512), 0, st, p);
  } else {
    set_grid<4, 1, 1>(p, grid);
    hipLaunchKernelGGL((fwd16_kernel<T, D, 4, 1, false, false, true>), grid, dim3(256), 0, st, p);
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
