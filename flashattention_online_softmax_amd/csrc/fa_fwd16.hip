// 16-bit (fp16 / bf16) attention forward kernels for gfx950, D in {64, 128}:
// dense, causal, boolean-masked, GQA and block-sparse.
//
// Method: the online-softmax forward of the "FlashAttention correctness
// verification" page (tiled computation and loop-invariant sections): per KV
// tile S = scale * Q K^T, a running row max m, l' = l e^(m - m') + rowsum
// e^(S - m'), O' = O e^(m - m') + e^(S - m') V, and finally O = O / l and
// LSE = m + ln l. The running max is moved with a rescale threshold in log2
// units (0 = exact running max; the lazy rescale of the flash-attention
// sparse-MLA page, threshold-branch section, for t > 0).
//
// This file is compiled on its own into a gfx950 code object (see build.py:
// the kernels keep the Q^T operands in 32 AGPRs and need the rest of a
// wave's 256 registers as VGPRs, a split the code object gets through its
// amdgpu-agpr-alloc attribute) and is
// loaded by the library at run time. Kernels are extern "C" with names of the
// form fa_fwd16_<dtype>_d<D>_w<waves>_h<heads>_c<causal>m<mask>s<sparse>.
//
// Work decomposition (MI355X): one workgroup of NW waves owns MPH consecutive
// query rows of HP query heads that share one KV head (HP > 1 packs GQA heads
// so that one K/V tile in LDS serves them all); every wave owns 32 query
// rows. With 8 waves two share each SIMD. Workgroups are numbered so that the
// longest causal row blocks start first and every KV head maps to one XCD.
//
// Per key tile (96 keys for dense D = 128, else 64) and wave:
//   * K and V tiles are copied HBM -> LDS by global_load_lds_dwordx4 (no
//     register staging) into three-deep rings, with an XOR swizzle of the
//     16-byte chunks so that the MFMA operand reads hit distinct LDS banks.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T
//     resident in AGPRs as the B operand). Each lane owns one query column
//     and 16 keys of it, so the row max and row sum are in-lane reductions
//     plus one v_permlane32_swap between the wave halves.
//   * p = exp2(s * scale*log2e - m) (one FMA + one v_exp_f32 per score), m
//     being the reference max already in the exp2 domain; l accumulates the
//     fp32 p; p is rounded to 16 bits into the B operand of the next MFMA.
//   * O^T += V^T P^T on MFMA with the accumulators in VGPRs: V^T is read from
//     the row-major V tile with ds_read_b64_tr_b16, in the key order in which
//     the S^T accumulator holds P. A rescale is one v_mul_f32 per
//     accumulator (in AGPRs it would be a read, a multiply and a write each,
//     which made the exact running max three times as expensive).
// Epilogue: O = acc / l rounded to the output dtype, LSE = ln2 * (m + log2 l)
// in fp32; rows with no key give O = 0 and LSE = -inf.
#include <stdint.h>

#include <type_traits>

#include "fa_asm.h"
#include "fa_copy.h"
#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// Per key tile j (BNT = 32 NKT keys: 96 for the dense D = 128 kernels
// without a boolean mask, 64 for the masked ones, for D = 64 and for the
// block-sparse ones, whose 128-key blocks split into two tiles) a wave (QT
// blocks of 32 query rows; every K/V operand it reads serves all of them)
// has a VALU phase V(j) and an MFMA phase M(j):
//   V(j): mask, row max, reference max update, p = exp2(s c - m), row sum,
//         p rounded into the P operand (and the rare rescale of O);
//   M(j): S(j+1) = K_{j+1} Q^T and O^T += V_j^T P_j^T, interleaved.
// The waves form two groups one phase apart (see the loop below), so on each
// SIMD one wave's V phase overlaps the other's M phase.
//
// Running max with a rescale threshold t (log2 units): a row's reference max
// moves only when the tile's max exceeds it by more than t; then O and l are
// rescaled by exp2(m_old - m_new). t = 0 is the exact running max (every
// growth rescales, the largest p of the row is exactly 1); t > 0 is the lazy
// rescale, with p <= 2^t.
//
// K and V tiles live in three-deep LDS rings (tile t in slot t % 3), filled
// by LDS-DMA copies issued three (K) and two (V) tiles ahead of use.
//
// XM = 1: packed variable-length batches (cu_q / cu_k give each batch's rows
// and keys); XM = 2: split-KV, the workgroup sweeps only the keys
// [split * split_len, (split + 1) * split_len) and writes its normalised fp32
// output and LSE to the partial-result buffers instead of O and LSE.
template <class T, int D, int NW, int QT, int HP, bool CAUSAL, int MASKM, bool SPARSE, int XM>
__device__ __forceinline__ void fwd16_body(const FwdParams& p) {
  // Boolean mask: MASKM = 1 loads each wave's mask words into registers one
  // phase ahead; MASKM = 2 copies each wave's mask rows into LDS two tiles
  // ahead with the K/V copies (16-byte aligned masks), with the keys of the
  // K and V tiles permuted (perm_key) so that a lane's 16 keys of a 32-key
  // half are consecutive and their mask bytes one 16-byte chunk.
  constexpr bool MASK = MASKM != 0;
  constexpr bool MLDS = MASKM == 2;
  constexpr int WPH = NW / HP;
  constexpr int MPH = WPH * QT * 32;
  // 32-key halves per tile: 3 for dense D = 128 without a boolean mask; the
  // masked kernels spend those registers on the prefetched mask words.
  constexpr int NKT = (SPARSE || MASK || D == 64) ? 2 : 3;
  constexpr int BNT = 32 * NKT;        // keys per tile
  constexpr int DS = D / 16;           // MFMA k-steps over D for S^T
  constexpr int DT = D / 32;           // 32-wide d tiles of O^T
  constexpr int NKS = 2 * NKT;         // 16-key steps per tile
  constexpr int NS = NKT * DS;         // K operands per tile (key halves x DS)
  constexpr int NP = NKS * DT;         // V operands per tile (key steps x DT)
  static_assert(NS == NP, "K and V operand counts agree (D / 8 each)");
  constexpr int TILE = BNT * D;
  constexpr int AHEAD = 3;    // operand pairs read ahead
  constexpr int RING = AHEAD + 1;
  static_assert(!SPARSE || MPH == 128, "block-sparse needs 128 query rows per head");
  static_assert(!MLDS || (QT == 1 && HP == 1 && BNT == 64), "LDS-staged masks: 32 rows per wave, 64-key tiles");

  // K ring (3 tiles) then V ring (3 tiles); the epilogue reuses the space.
  __shared__ __attribute__((aligned(16))) uint16_t s_ring[6 * TILE];
  uint16_t* const s_kring = s_ring;
  uint16_t* const s_vring = s_ring + 3 * TILE;
  __shared__ int s_kstart[SPARSE ? 512 : 1];
  // LDS-staged mask tiles: per wave three slots of its 32 rows x 64 bytes,
  // 16-byte chunk c of row r at chunk position c ^ ((r >> 2) & 3) (the
  // chunk reads of 16 consecutive rows then hit distinct banks).
  constexpr int MSLOT = 32 * BNT;
  __shared__ __attribute__((aligned(16))) uint8_t s_mring[MLDS ? NW * 3 * MSLOT : 16];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;
  Work wk = decode_work<NW, QT, HP, XM>(p);
  const int diag = wk.Lk - wk.Lq;  // key j is visible to row i iff j <= i + diag
  // First key of this workgroup's range; under split-KV its range ends at
  // wk.Lk (keys from there on are masked like keys past the sequence).
  int klo = 0;
  if (XM == 2) {
    klo = wk.split * p.split_len;
    wk.Lk = min(wk.Lk, klo + p.split_len);
  }
  // Rows of this head: Sq, or the batch's own length in the packed layout.
  const int rlim = XM == 1 ? wk.Lq : p.Sq;
  if constexpr (XM == 0) {
    // A query block wholly past the batch's length: its rows (padding up to
    // Sq) get O = 0 and LSE = -inf without the tile pipeline.
    if (wk.wg_row0 >= wk.Lq) {
      constexpr int CPR = D / 8, RPI = 64 / CPR;  // 16-byte chunks per row, rows per store
      uint16_t* og0 = (uint16_t*)p.o + wk.b * p.o_sb + wk.hq * p.o_sh;
#pragma unroll
      for (int k = 0; k < QT * 32 / RPI; ++k) {
        const int qrow = wk.row0 + k * RPI + lane / CPR;
        if (qrow < p.Sq) *(u32x4*)(og0 + (int64_t)qrow * p.o_ss + 8 * (lane % CPR)) = u32x4{0u, 0u, 0u, 0u};
      }
      if (p.o_lo) {
        constexpr int FPR = D / 4, FRI = 64 / FPR;  // float4 per o_lo row, rows per store
        float* l0 = p.o_lo + wk.b * p.ol_sb + wk.hq * p.ol_sh;
#pragma unroll
        for (int k = 0; k < QT * 32 / FRI; ++k) {
          const int qrow = wk.row0 + k * FRI + lane / FPR;
          if (qrow < p.Sq) *(float4*)(l0 + (int64_t)qrow * p.ol_ss + 4 * (lane % FPR)) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int b = 0; b < QT; ++b) {
        const int qrow = wk.row0 + 32 * b + c;
        if (h == 0 && qrow < p.Sq) p.lse[wk.b * p.lse_sb + wk.hq * p.lse_sh + (int64_t)qrow * p.lse_ss] = -INFINITY;
      }
      return;
    }
  }

  int n_iter;
  if (SPARSE)
    n_iter = build_sparse_tiles(p, wk, wk.wg_row0 / 128, s_kstart, &s_n);
  else
    n_iter = dense_tiles<CAUSAL>(wk, MPH, BNT, diag, klo);
  // Tiles this wave works on: none if its rows are past Lq; under the causal
  // mask only the tiles that start at or before its last visible key.
  int n_act = n_iter;
  if (wk.row0 >= wk.Lq) {
    n_act = 0;
  } else if (CAUSAL && !SPARSE) {
    const int last_key = min(wk.row0 + QT * 32 - 1, wk.Lq - 1) + diag;
    n_act = last_key < klo ? 0 : min(n_iter, (last_key - klo) / BNT + 1);
  }
  n_act = __builtin_amdgcn_readfirstlane(n_act);

  const uint16_t* qg = (const uint16_t*)p.q + wk.b * p.q_sb + wk.hq * p.q_sh + (int64_t)wk.qoff * p.q_ss;
  const uint16_t* kg = (const uint16_t*)p.k + wk.b * p.k_sb + wk.hkv * p.k_sh + (int64_t)wk.koff * p.k_ss;
  const uint16_t* vg = (const uint16_t*)p.v + wk.b * p.v_sb + wk.hkv * p.v_sh + (int64_t)wk.koff * p.v_ss;

  u32x4 qop[QT][DS];  // Q^T operands, loaded after the first tile copies

  f32x16 oacc[QT][DT];
#pragma unroll
  for (int b = 0; b < QT; ++b)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][dt][i] = 0.f;
#pragma unroll
  for (int b = 0; b < QT; ++b) vacc_written(oacc[b]);
  float m_ref[QT], l_run[QT];
  f32x16 sc[QT][NKT];    // [block][kt]: scores of the tile the next softmax works on
  u32x4 pp[1][QT][NKS];  // P operand of the tile between its V and M phases
#pragma unroll
  for (int b = 0; b < QT; ++b) {
    m_ref[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[b][kt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pp[0][b][ks] = u32x4{0u, 0u, 0u, 0u};
  }

  auto tile_start = [&](int it) __attribute__((always_inline)) { return SPARSE ? s_kstart[it] : klo + it * BNT; };

  const TileCopy<D, NW, false, BNT, MLDS> kcopy(kg, p.k_ss);
  const TileCopy<D, NW, true, BNT, MLDS> vcopy(vg, p.v_ss);
  constexpr int MCOPY = MLDS ? MSLOT / 1024 : 0;  // mask copy instructions per wave and tile
  constexpr int NCOPY = TileCopy<D, NW, false, BNT, MLDS>::PER_WAVE + TileCopy<D, NW, true, BNT, MLDS>::PER_WAVE + MCOPY;

  // Per-lane element offsets of the MFMA operands inside a tile.
  // K operand r (A operand of S^T): key half kt = r % NKT (rows 32 kt + c),
  // logical chunk 2 (r / NKT) + h.
  int koff[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = c * D + (((2 * ds + h) ^ kswz<D>(c)) << 3);
  // V operand r (tr-read, see lds_read_tr16): key step ks = r / DT (keys
  // 16 ks .. +15, lane rows vrow and vrow + 8), d tile dt = r % DT.
  const int vrow = 4 * h + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int voff[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int col = 32 * dt + vcol;
    voff[dt] = vrow * D + (((col >> 3) ^ vswz<D>(vrow)) << 3) + (col & 7);
  }
  auto kread = [&](const lds_u16* kb, int r) __attribute__((always_inline)) -> u32x4 {
    return *(const __attribute__((address_space(3))) u32x4*)(kb + (r % NKT) * 32 * D + koff[r / NKT]);
  };
  auto vread = [&](const lds_u16* const (&vb)[DT], int r) __attribute__((always_inline)) -> u32x4 {
    const int dt = r % DT, ks = r / DT;
    const int rb = ((ks >> 1) * 32 + (ks & 1) * 16) * D;  // vswz depends on row % 4 only
    const u32x2 lo = lds_read_tr16(vb[dt] + rb);
    const u32x2 hi = lds_read_tr16(vb[dt] + rb + 8 * D);
    const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return v;
  };

  // Masking of tile j's scores of block b (causal diagonal, ragged edges,
  // boolean mask).
  // Boolean-mask words of the tile the next V phase masks, per block: 4 mask
  // bytes (keys 8 g + 4 h .. +3 of key half kt of the lane's row). They are
  // loaded at the start of the M phase before that V phase, so the global
  // load latency hides behind its MFMAs, and are pinned in registers before
  // the phase's tile copies go out (a later wait for them would also drain
  // the copies).
  uint32_t mwords[QT][MASK ? NKT : 1][4];
  auto mask_load = [&](int j) __attribute__((always_inline)) {
    if constexpr (MASK && !MLDS) {
      const int kstart = tile_start(j);
      if (NKT == 2 && p.mask_vec16 && kstart + BNT <= p.Skv) {
        // Coalesced: the two lanes of a row load its 64 mask bytes, 32 each
        // (lane half h: bytes 32 h .. 32 h + 31, own words 0..7 = row words
        // 8 h .. 8 h + 7), then trade words across the wave halves. Word
        // 8 kt + 2 g + h is what mwords[kt][g] needs: swapping the upper half
        // of own word 2 g with the lower half of own word 2 g + 1 gives the
        // kt = 0 word in the first result and the kt = 1 word in the second,
        // on both halves.
#pragma unroll
        for (int b = 0; b < QT; ++b) {
          const int qrow = wk.row0 + 32 * b + c;
          u32x4 lo = {0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u}, hi = lo;
          if (qrow < p.Sq) {
            const u32x4* src = (const u32x4*)(p.mask + wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)qrow * p.m_ss +
                                              kstart + 32 * h);
            lo = src[0];
            hi = src[1];
          }
          const uint32_t own[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const auto r = __builtin_amdgcn_permlane32_swap(own[2 * g], own[2 * g + 1], false, false);
            mwords[b][0][g] = r[0];
            mwords[b][NKT - 1][g] = r[1];
          }
        }
        return;
      }
      const bool vec = p.mask_vec4 && (kstart + BNT <= p.Skv);
#pragma unroll
      for (int b = 0; b < QT; ++b) {
        const int qrow = wk.row0 + 32 * b + c;
        const uint8_t* mrow = p.mask + wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)qrow * p.m_ss;
        const bool rv = qrow < p.Sq;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
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
            mwords[b][kt][g] = bits;
          }
      }
    }
  };
  // LDS-staged masks: lane i of copy instruction n fetches chunk position
  // 64 n + i of the wave's slot (row r = pos / 4). Rows past Sq fetch row
  // Sq - 1 and chunks at or past Skv the row's last chunk: finite bytes
  // whose keys or rows the edge masking removes.
  const int mrow_b = min(wk.row0, p.Sq - 1);
  const uint8_t* const mbase =
      MLDS ? p.mask + wk.b * p.m_sb + wk.hq * p.m_sh + (int64_t)mrow_b * p.m_ss : nullptr;
  uint32_t mroff[MCOPY > 0 ? MCOPY : 1];
  int mcol[MCOPY > 0 ? MCOPY : 1];
#pragma unroll
  for (int n = 0; n < MCOPY; ++n) {
    const int pos = 64 * n + lane, r = pos >> 2;
    mroff[n] = (uint32_t)(min(wk.row0 + r, p.Sq - 1) - mrow_b) * (uint32_t)p.m_ss;
    mcol[n] = 16 * ((pos & 3) ^ ((r >> 2) & 3));
  }
  const int wv = (int)threadIdx.x >> 6;
  auto mslot = [&](int j) __attribute__((always_inline)) -> uint8_t* { return s_mring + (wv * 3 + j % 3) * MSLOT; };
  auto mask_copy = [&](int j) __attribute__((always_inline)) {
    if constexpr (MLDS) {
      const int kstart = __builtin_amdgcn_readfirstlane(tile_start(j));
      const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr_of(mslot(j)));
#pragma unroll
      for (int n = 0; n < MCOPY; ++n)
        lds_copy16(mbase + kstart, mroff[n] + (uint32_t)min(mcol[n], p.Skv - 16 - kstart), l0 + n * 1024);
    }
  };
  // Mask words of tile j from LDS: key half kt of the lane's row is chunk
  // 2 kt + h (keys 32 kt + 16 h .. +15 in the permuted tile layout).
  auto mask_read = [&](int j) __attribute__((always_inline)) {
    if constexpr (MLDS) {
      const uint8_t* row = mslot(j) + c * BNT;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const u32x4 w = *(const __attribute__((address_space(3))) u32x4*)lds_ptr(
            lds_addr_of(row) + 16 * ((2 * kt + h) ^ ((c >> 2) & 3)));
#pragma unroll
        for (int g = 0; g < 4; ++g) mwords[0][kt][g] = w[g];
      }
    }
  };
  auto mask_pin = [&]() __attribute__((always_inline)) {
    if constexpr (MASK) {
#pragma unroll
      for (int b = 0; b < QT; ++b)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) asm volatile("" ::"v"(mwords[b][kt][g]));
    }
  };

  // Masking of tile j's scores of block b (causal diagonal, ragged edges,
  // boolean mask from mwords).
  auto mask_tile = [&](f32x16 (&sv)[NKT], int b, int j) __attribute__((always_inline)) {
    const int kstart = tile_start(j);
    const int brow0 = wk.row0 + 32 * b;
    const int qrow = brow0 + c;
    const bool edge = (kstart + BNT > wk.Lk) || (brow0 + 32 > wk.Lq) ||
                      (CAUSAL && kstart + BNT - 1 > brow0 + diag);
    if constexpr (MASK) {
      if (!edge) {  // inside every range: the mask bytes alone decide
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (((mwords[b][kt][i >> 2] >> (8 * (i & 3))) & 0xffu) != 0u) sv[kt][i] = -INFINITY;
        return;
      }
    } else if (!edge) {
      return;
    }
    // The lane's last visible key (-1: none): keys of its row run up to
    // Lk - 1, and under the causal mask up to qrow + diag; rows past Lq see
    // none. lim_lo is the smallest of these over the block's 32 rows (the
    // first row's under the causal mask), the same in every lane.
    int lim = qrow < wk.Lq ? wk.Lk - 1 : -1;
    if (CAUSAL) lim = min(lim, qrow + diag);
    int lim_lo = brow0 + 32 <= wk.Lq ? wk.Lk - 1 : -1;
    if (CAUSAL) lim_lo = min(lim_lo, brow0 + diag);
    lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int k0 = kstart + kt * 32;
      // Key half kt entirely visible in every row: only the mask bytes apply.
      if (!MASK && k0 + 31 <= lim_lo) continue;
      // Element i holds key k0 + 4 h + 8 (i / 4) + i % 4 (permuted tiles:
      // k0 + 16 h + i): visible iff 8 (i / 4) + i % 4 <= r (i <= r).
      const int r = k0 + 31 <= lim_lo ? 31 : lim - k0 - (MLDS ? 16 : 4) * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bool ok = (MLDS ? i : 8 * (i >> 2) + (i & 3)) <= r;
        if constexpr (MASK) ok = ok && ((mwords[b][kt][i >> 2] >> (8 * (i & 3))) & 0xffu) == 0u;
        if (!ok) sv[kt][i] = -INFINITY;
      }
    }
  };

  // Softmax state of the step being processed, per block.
  float mq[QT], mc[QT], alpha[QT], rs0[QT], rs1[QT];
  bool upd_any = false;
  // Part (0 .. 2 NKT - 1, 8 scores each) of block b's row max (three-input
  // maxima).
  auto row_max_4 = [&](const f32x16 (&sv)[NKT], int b, int part) __attribute__((always_inline)) {
    const int kt = part >> 1, i0 = (part & 1) * 8;
    const float t = max3(sv[kt][i0], sv[kt][i0 + 1], sv[kt][i0 + 2]);
    const float u = max3(t, sv[kt][i0 + 3], sv[kt][i0 + 4]);
    const float v = max3(u, sv[kt][i0 + 5], sv[kt][i0 + 6]);
    mq[b] = part == 0 ? fmaxf(v, sv[kt][i0 + 7]) : max3(mq[b], v, sv[kt][i0 + 7]);
    asm volatile("" ::"v"(mq[b]));
  };
  // Reference-max update of block b. An inactive step (no tile of this wave)
  // leaves m alone; below n_iter its scores come from real K rows, are finite,
  // and give P = 0 for the P V of the next step; the last step's P is never
  // used.
  auto max_update = [&](int b, bool act) __attribute__((always_inline)) {
    const float mx = half_max(mq[b]) * p.scale_log2;
    const bool upd = act && mx > m_ref[b] + p.rescale_thr;
    const float m_new = upd ? mx : m_ref[b];
    alpha[b] = upd ? fast_exp2(m_ref[b] - m_new) : 1.f;
    upd_any = upd_any || upd;
    m_ref[b] = m_new;
    mc[b] = !act ? INFINITY : (m_new == -INFINITY ? 0.f : m_new);
    rs0[b] = 0.f;
    rs1[b] = 0.f;
  };
  // Exponentials of block b's scores e, e+1 (e even) into its P operand.
  auto exp_pair = [&](const f32x16 (&sv)[NKT], u32x4 (&pop)[NKS], int b, int e) __attribute__((always_inline)) {
    const int kt = e >> 4, ii = e & 15;
    const float x0 = fast_exp2(__builtin_fmaf(sv[kt][ii], p.scale_log2, -mc[b]));
    const float x1 = fast_exp2(__builtin_fmaf(sv[kt][ii + 1], p.scale_log2, -mc[b]));
    pop[e >> 3][(e & 7) >> 1] = T::pack2(x0, x1);
    // two running sums (pairs alternate), each started by its first pair
    if ((e >> 1) & 1)
      rs1[b] = e == 2 ? x0 + x1 : rs1[b] + (x0 + x1);
    else
      rs0[b] = e == 0 ? x0 + x1 : rs0[b] + (x0 + x1);
    // Pin the results here: otherwise the compiler sinks the exponentials
    // below the MFMAs they are meant to overlap.
    asm volatile("" ::"v"(pop[e >> 3][(e & 7) >> 1]), "v"(rs0[b]), "v"(rs1[b]));
  };
  // Softmax slice s of a step (0 .. (10 NKT + 1) QT - 1): block maxima,
  // updates, then exponential pairs alternating between blocks.
  constexpr int NMAX = 2 * NKT;  // row-max parts per block
  constexpr int NSLICE = (5 * NMAX + 1) * QT;
  auto slice = [&](f32x16 (&sv)[QT][NKT], u32x4 (&pop)[QT][NKS], int s, bool act) __attribute__((always_inline)) {
    if (s < NMAX * QT) {
      row_max_4(sv[s / NMAX], s / NMAX, s % NMAX);
    } else if (s < (NMAX + 1) * QT) {
      max_update(s - NMAX * QT, act);
    } else {
      const int t = s - (NMAX + 1) * QT;  // 0 .. 8 NKT QT - 1
      const int b = t % QT, e = 2 * (t / QT);
      exp_pair(sv[b], pop[b], b, e);
    }
  };

  // M phase: S = K Q^T of the tile in kt_buf into sn and O^T += V^T P^T
  // with the tile in vt_buf, interleaved operand by operand (independent
  // accumulators), operands read AHEAD ahead.
  // Operands 0 .. AHEAD-1 of an M phase, read ahead of it (at the end of the
  // wave's V phase, so the M phase starts without waiting on LDS).
  u32x4 kq[RING], vq[RING];
  auto mprefetch = [&](const uint16_t* kt_buf, const uint16_t* vt_buf, bool do_pv) __attribute__((always_inline)) {
    const lds_u16* kb = lds_ptr(lds_addr_of(kt_buf));
    const lds_u16* vb[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vb[dt] = lds_ptr(lds_addr_of(vt_buf) + 2 * voff[dt]);
#pragma unroll
    for (int r = 0; r < AHEAD; ++r) {
      kq[r] = kread(kb, r);
      if (do_pv) vq[r] = vread(vb, r);
    }
  };
  auto mphase = [&](f32x16 (&sn)[QT][NKT], const u32x4 (&pop)[QT][NKS], const uint16_t* kt_buf,
                    const uint16_t* vt_buf, bool do_pv) __attribute__((always_inline)) {
    const lds_u16* kb = lds_ptr(lds_addr_of(kt_buf));
    const lds_u16* vb[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vb[dt] = lds_ptr(lds_addr_of(vt_buf) + 2 * voff[dt]);
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      if (r + AHEAD < NS) {
        kq[(r + AHEAD) % RING] = kread(kb, r + AHEAD);
        if (do_pv) vq[(r + AHEAD) % RING] = vread(vb, r + AHEAD);
      }
#pragma unroll
      for (int b = 0; b < QT; ++b) {
        // S: key half r % NKT, k-step r / NKT
        if (r < NKT)
          Mma<T>::v0b(sn[b][r % NKT], kq[r % RING], qop[b][r / NKT]);
        else
          Mma<T>::vb(sn[b][r % NKT], kq[r % RING], qop[b][r / NKT]);
        // P V: d tile r % DT, key step r / DT
        if (do_pv) Mma<T>::v(oacc[b][r % DT], vq[r % RING], pop[b][r / DT]);
      }
    }
    // S results complete before the compiler may touch the registers again.
#pragma unroll
    for (int b = 0; b < QT; ++b) mfma_wait_v(sn[b]);
  };

  // V phase: softmax(j) of the scores in sv into pop (VALU only), and the
  // rescale of O and l when a reference max moved (O is only ever touched by
  // MFMAs otherwise).
  auto vphase = [&](f32x16 (&sv)[QT][NKT], u32x4 (&pop)[QT][NKS], bool act, bool o_live)
                    __attribute__((always_inline)) {
    upd_any = false;
#pragma unroll
    for (int sl = 0; sl < NSLICE; ++sl) slice(sv, pop, sl, act);
    if (o_live && __builtin_amdgcn_ballot_w64(upd_any) != 0) {
#pragma unroll
      for (int b = 0; b < QT; ++b) {
        mfma_wait_v(oacc[b]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[b][dt][i] *= alpha[b];
        vacc_written(oacc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < QT; ++b) l_run[b] = act ? __builtin_fmaf(l_run[b], alpha[b], rs0[b] + rs1[b]) : l_run[b];
  };

  // Copies of K_{m+3} (into K_m's slot) and V_{m+2} (into V_{m-1}'s slot).
  auto copies = [&](int m) __attribute__((always_inline)) {
    bool any = false;
    if (m + 3 < n_iter) {
      kcopy.issue(tile_start(m + 3), wk.Lk, s_kring + (m % 3) * TILE);
      any = true;
    }
    if (m + 2 < n_iter) {
      vcopy.issue(tile_start(m + 2), wk.Lk, s_vring + ((m + 2) % 3) * TILE);
      mask_copy(m + 2);
      any = true;
    }
    return any;
  };
  // End of a phase: this wave's copies of the phase before are complete (those
  // of this phase may still fly), then the workgroup barrier.
  auto end_phase = [&](bool copied_now) __attribute__((always_inline)) {
    if (copied_now)
      wait_vmem_below<NCOPY>();
    else
      wait_vmem();
    barrier_keep_copies();
  };

  // Prologue: K_0, K_1, K_2, V_0, V_1 in flight.
  if (n_iter > 0) {
    kcopy.issue(tile_start(0), wk.Lk, s_kring);
    vcopy.issue(tile_start(0), wk.Lk, s_vring);
    mask_copy(0);
  }
  if (n_iter > 1) {
    kcopy.issue(tile_start(1), wk.Lk, s_kring + TILE);
    vcopy.issue(tile_start(1), wk.Lk, s_vring + TILE);
    mask_copy(1);
  }
  if (n_iter > 2) kcopy.issue(tile_start(2), wk.Lk, s_kring + 2 * TILE);
  // Q^T operands (B operand of S^T = K Q^T, kept in AGPRs): block b, lane
  // holds Q[row0 + 32 b + c][16 ds + 8 h .. +7]. Loaded after the copies are
  // issued so that both latencies overlap.
#pragma unroll
  for (int b = 0; b < QT; ++b) {
    const int qrow = wk.row0 + 32 * b + c;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qrow < rlim) z = *(const u32x4*)(qg + (int64_t)qrow * p.q_ss + 16 * ds + 8 * h);
      qop[b][ds] = z;
    }
  }
  // Make the compiler wait for the Q loads here, once: it does not see the
  // copies above, and otherwise would wait for its Q loads (vmcnt(0), which
  // drains copies in flight) at their first use inside the loop.
#pragma unroll
  for (int b = 0; b < QT; ++b)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) asm volatile("s_nop 4" : "+a"(qop[b][ds]));
  wait_vmem();
  __syncthreads();

  // Two wave groups one phase apart: group 0 runs M(-1) V(0) M(0) V(1) ...,
  // group 1 the same one phase later; every phase ends with a workgroup
  // barrier. Waves w and w + NW/2 share a SIMD, so there one wave's softmax
  // issues while the other's MFMAs run. M(j) computes S(j+1) and O += P(j)
  // V(j); V(j) turns S(j) into P(j). Every wave runs the same stream: a
  // softmax past this wave's tiles is inactive (P = 0, m and l unchanged),
  // and the S of the last M phase is computed from a slot whose result goes
  // unused.
  //
  // Copies: every wave issues its share of the copies of K_{j+3} (into K_j's
  // slot) and V_{j+2} (into V_{j-1}'s slot) right after the MFMAs of its
  // M(j), while they drain. Those slots were last read in M(j-1), which both
  // groups have finished (group 0's M(j) is global phase 2j+2, group 1's
  // M(j-1) is 2j+1). A wave waits for its copies at the end of its next
  // phase; the first reader of K_{j+3} / V_{j+2} is M(j+2), two phases later.
  const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) / (NW / 2));
  if (grp == 1) end_phase(false);
  if (n_act > 0) {
    mask_load(0);
    mask_read(0);
  }
  mprefetch(s_kring, s_vring, false);
  mphase(sc, pp[0], s_kring, s_vring, false);  // M(-1): S(0)
  mask_pin();
  end_phase(false);
  for (int j = 0; j < n_iter; ++j) {
    const bool act = j < n_act;
    const uint16_t* kt_buf = s_kring + ((j + 1) % 3) * TILE;  // K_{j+1}
    const uint16_t* vt_buf = s_vring + (j % 3) * TILE;        // V_j
    // V(j): global phase 2j+1 (group 0) or 2j+2 (group 1).
    if (act) {
#pragma unroll
      for (int b = 0; b < QT; ++b) mask_tile(sc[b], b, j);
    }
    vphase(sc, pp[0], act, j > 0);
    // K_{j+1} and V_j have been in LDS since phase 2j (their copies were
    // waited for two phases after they were issued in M(j-2)).
    mprefetch(kt_buf, vt_buf, true);
    end_phase(false);
    // M(j): global phase 2j+2 (group 0) or 2j+3 (group 1).
    if (j + 1 < n_act) mask_load(j + 1);
    mphase(sc, pp[0], kt_buf, vt_buf, true);
    // Mask tile j+1 has been in LDS since the end of V(j) (this wave's own
    // copies, issued in M(j-1), are waited for there).
    if (j + 1 < n_act) mask_read(j + 1);
    mask_pin();
    end_phase(copies(j));
  }
  if (grp == 0) end_phase(false);

  // Epilogue: O = acc / l rounded to the output dtype, staged through LDS
  // (free now: every wave is past its last ring read and copy) so that each
  // store instruction writes whole rows, 16 bytes per lane; LSE = ln2 (m +
  // log2 l) in fp32. Rows with no key give O = 0 and LSE = -inf.
  if constexpr (XM == 2) {
    // Split-KV: this key range's normalised fp32 output and LSE (natural
    // log; -inf and zeros when the range has no visible key) for the merge.
    const int64_t rbase = (int64_t)wk.split * ((int64_t)p.B * p.Hq * p.Sq) + ((int64_t)wk.b * p.Hq + wk.hq) * p.Sq;
#pragma unroll
    for (int b = 0; b < QT; ++b) {
      mfma_wait_v(oacc[b]);
      const int qrow = wk.row0 + 32 * b + c;
      const float lt = half_sum(l_run[b]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (qrow < p.Sq) {
        float* dst = p.part_o + (rbase + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(float4*)(dst + 32 * dt + 8 * g + 4 * h) =
                make_float4(oacc[b][dt][4 * g] * inv, oacc[b][dt][4 * g + 1] * inv, oacc[b][dt][4 * g + 2] * inv,
                            oacc[b][dt][4 * g + 3] * inv);
        if (h == 0) p.part_lse[rbase + qrow] = lt > 0.f ? (m_ref[b] + log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    return;
  }
  constexpr int OPAD = D + 8;  // padded LDS row: a 16-byte bank shift per row
  static_assert(NW * QT * 32 * OPAD <= 6 * TILE, "O staging fits in the rings");
  uint16_t* const s_o = s_ring + ((int)threadIdx.x >> 6) * (QT * 32 * OPAD);
  uint16_t* og = (uint16_t*)p.o + wk.b * p.o_sb + wk.hq * p.o_sh + (int64_t)wk.qoff * p.o_ss;
  // With o_lo, the fp32 residual O - rounded(O) of each element goes to HBM
  // straight from the registers (4 consecutive columns per lane and store).
  float* const olo = p.o_lo ? p.o_lo + wk.b * p.ol_sb + wk.hq * p.ol_sh + (int64_t)wk.qoff * p.ol_ss : nullptr;
#pragma unroll
  for (int b = 0; b < QT; ++b) {
    mfma_wait_v(oacc[b]);
    const int qrow = wk.row0 + 32 * b + c;
    const float lt = half_sum(l_run[b]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = s_o + (32 * b + c) * OPAD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float x0 = oacc[b][dt][4 * g] * inv, x1 = oacc[b][dt][4 * g + 1] * inv;
        const float x2 = oacc[b][dt][4 * g + 2] * inv, x3 = oacc[b][dt][4 * g + 3] * inv;
        u32x2 v;
        v[0] = T::pack2(x0, x1);
        v[1] = T::pack2(x2, x3);
        *(u32x2*)(orow + 32 * dt + 8 * g + 4 * h) = v;
        if (olo && qrow < rlim) {
          const f32x2 r0 = T::unpack2(v[0]), r1 = T::unpack2(v[1]);
          *(float4*)(olo + (int64_t)qrow * p.ol_ss + 32 * dt + 8 * g + 4 * h) =
              make_float4(x0 - r0[0], x1 - r0[1], x2 - r1[0], x3 - r1[1]);
        }
      }
    if (h == 0 && qrow < rlim)
      p.lse[wk.b * p.lse_sb + wk.hq * p.lse_sh + (int64_t)(wk.qoff + qrow) * p.lse_ss] =
          lt > 0.f ? (m_ref[b] + log2f(lt)) * kLn2 : -INFINITY;
  }
  // The wave reads back what its own lanes wrote (LDS operations of a wave
  // complete in order).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;     // rows per store instruction
#pragma unroll
  for (int k = 0; k < QT * 32 / RPI; ++k) {
    const int r = k * RPI + lane / CPR, ch = lane % CPR;
    const int qrow = wk.row0 + r;
    const u32x4 v = *(const u32x4*)(s_o + r * OPAD + 8 * ch);
    if (qrow < rlim) *(u32x4*)(og + (int64_t)qrow * p.o_ss + 8 * ch) = v;
  }
}

}  // namespace
}  // namespace fa

// Kernel entry points (names are looked up by the library at run time):
// fa_fwd16_<dtype>_d<D>_w<waves>_q<32-row blocks per wave>_h<heads>_c<causal>m<mask>s<sparse>x<mode>,
// mode 0 = BNSD, 1 = packed variable-length batches, 2 = split-KV partials.
#define FA_FWD16_KERNEL(TN, T, D, NW, QT, HP, C, M, S, X)                                              \
  extern "C" __global__ void __launch_bounds__(NW * 64, 1)                                             \
      fa_fwd16_##TN##_d##D##_w##NW##_q##QT##_h##HP##_c##C##m##M##s##S##x##X(const fa::FwdParams p) {  \
    fa::fwd16_body<fa::T, D, NW, QT, HP, C != 0, M, S != 0, X>(p);                                      \
  }
#define FA_FWD16_DTYPE_D(TN, T, D)                    \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 0, 0, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 0, 1, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 1, 0, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 1, 1, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 0, 2, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 1, 2, 0, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 2, 0, 0, 1, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 4, 1, 1, 0, 0, 1, 0)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 0, 0, 0, 1)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 1, 0, 0, 1)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 0, 0, 0, 2)      \
  FA_FWD16_KERNEL(TN, T, D, 8, 1, 1, 1, 0, 0, 2)

FA_FWD16_DTYPE_D(f16, F16, 64)
FA_FWD16_DTYPE_D(f16, F16, 128)
FA_FWD16_DTYPE_D(bf16, BF16, 64)
FA_FWD16_DTYPE_D(bf16, BF16, 128)
