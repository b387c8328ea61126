// HBM -> LDS tile copies of the 16-bit attention kernels (LDS-DMA, no
// register staging), in the chunk-swizzled tile layout of fa_tiles.h.
#pragma once

#include <stdint.h>

#include "fa_asm.h"
#include "fa_tiles.h"

namespace fa {

// Copies of ROWS-key tiles (rows kstart .. kstart+ROWS-1 of one K or V head)
// into LDS buffers of ROWS rows x D elements stored with the 16-byte chunk
// swizzle.
// One copy instruction fills 64 consecutive chunks (1 KB) of LDS, lane i
// chunk 64n + i, so each lane fetches the logical chunk the swizzle keeps at
// that position (the XOR is an involution). The per-lane byte offset inside a
// tile is the same for every tile and is computed once. On the last, partial
// tile, rows at or past Lk fetch row Lk - 1 instead (finite data whose scores
// are masked), so nothing past the valid keys is ever read. With PERM, LDS
// row r of the tile receives key perm_key(r) instead of key r.
template <int D, int NW, bool IS_V, int ROWS = BN, bool PERM = false>
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int NINST = ROWS * CH / 64;
  static constexpr int PER_WAVE = NINST / NW;
  static_assert(NINST % NW == 0, "tile copy must divide evenly over the waves");
  const char* g;       // head base
  uint32_t row_bytes;  // row stride in bytes (the library keeps it below 2^24)
  uint32_t off[PER_WAVE];

  __device__ __forceinline__ static int pos(int j) {
    return (((int)threadIdx.x >> 6) * PER_WAVE + j) * 64 + ((int)threadIdx.x & 63);
  }
  __device__ __forceinline__ static int chunk_row(int j) { return pos(j) / CH; }
  // Key (row of the K or V head, from the tile start) that LDS row chunk_row(j) holds.
  __device__ __forceinline__ static int src_row(int j) { return PERM ? perm_key(chunk_row(j)) : chunk_row(j); }
  __device__ __forceinline__ static uint32_t chunk_col_bytes(int j) {
    const int row = pos(j) / CH, ph = pos(j) % CH;
    return (uint32_t)((ph ^ (IS_V ? vswz<D>(row) : kswz<D>(row))) * 16);
  }

  // head is the same in every lane of the wave.
  __device__ __forceinline__ TileCopy(const uint16_t* head, int64_t row_stride)
      : g(uniform_ptr(head)), row_bytes((uint32_t)row_stride * 2u) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) off[j] = (uint32_t)src_row(j) * row_bytes + chunk_col_bytes(j);
  }

  // kstart, Lk and lds are the same in every lane of the wave.
  __device__ __forceinline__ void issue(int kstart, int Lk, const uint16_t* lds) const {
    kstart = __builtin_amdgcn_readfirstlane(kstart);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(
        lds_addr_of(lds) + (((int)threadIdx.x >> 6) * PER_WAVE) * 1024);
    const char* base = g + (int64_t)kstart * row_bytes;
    if (kstart + ROWS <= Lk) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) lds_copy16(base, off[j], l0 + j * 1024);
    } else {
      const int last = Lk - 1 - kstart;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int over = max(src_row(j) - last, 0);
        lds_copy16(base, off[j] - (uint32_t)over * row_bytes, l0 + j * 1024);
      }
    }
  }
};

}  // namespace fa
