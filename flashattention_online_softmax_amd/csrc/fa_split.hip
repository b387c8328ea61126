// Merge of the split-KV partial results into the attention output.
//
// Each key range s of a row produced an output O_s normalised by its own row
// sum and the natural-log LSE_s of its scores (LSE_s = -inf, O_s = 0 when the
// range holds no visible key). The whole row's result is the combination of
// partial softmax states described on the "FlashAttention correctness
// verification" page (standard vs tiled attention: per-block max and sum,
// merged by rescaling to the common max), written with the LSE:
//   LSE = M + ln sum_s exp(LSE_s - M),   M = max_s LSE_s
//   O   = sum_s exp(LSE_s - LSE) O_s
// A row with no visible key in any range gets O = 0 and LSE = -inf.
//
// Memory-bound: one wave per row, each lane owns Dv / 64 consecutive columns;
// reads n_splits (Dv + 1) fp32 values per row and writes one 16-bit row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Static partial-result buffer of the allocation-free split-KV entry point:
// every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory; the
// device address comes from hipGetSymbolAddress, once per device (below).
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

constexpr int kRowsPerBlock = 4;

template <class T, int DV>
__global__ __launch_bounds__(64 * kRowsPerBlock) void splitkv_merge_kernel(const MergeParams p) {
  constexpr int C = DV / 64;  // columns per lane (1 or 2)
  const int lane = threadIdx.x & 63;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= nrows) return;
  float mx = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) mx = fmaxf(mx, p.part_lse[(int64_t)s * nrows + row]);
  float acc[C];
#pragma unroll
  for (int e = 0; e < C; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < p.n_splits; ++s) {
      const float ls = p.part_lse[(int64_t)s * nrows + row];
      const float w = ls == -INFINITY ? 0.f : fast_exp2((ls - mx) * 1.4426950408889634f);
      wsum += w;
      const float* src = p.part_o + ((int64_t)s * nrows + row) * DV + C * lane;
#pragma unroll
      for (int e = 0; e < C; ++e) acc[e] = __builtin_fmaf(w, src[e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t i = row % p.Sq, bh = row / p.Sq, hq = bh % p.Hq, b = bh / p.Hq;
  uint16_t* dst = (uint16_t*)p.o + b * p.o_sb + hq * p.o_sh + i * p.o_ss + C * lane;
  if constexpr (C == 2) {
    *(uint32_t*)dst = T::pack2(acc[0] * inv, acc[1] * inv);
  } else {
    const uint32_t w2 = T::pack2(acc[0] * inv, 0.f);
    *dst = (uint16_t)(w2 & 0xffffu);
  }
  if (lane == 0) p.lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

template <class T>
hipError_t launch_merge_t(const MergeParams& m, hipStream_t st) {
  const int64_t nrows = (int64_t)m.B * m.Hq * m.Sq;
  const dim3 grid((unsigned)((nrows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (m.Dv == 128)
    hipLaunchKernelGGL((splitkv_merge_kernel<T, 128>), grid, dim3(64 * kRowsPerBlock), 0, st, m);
  else
    hipLaunchKernelGGL((splitkv_merge_kernel<T, 64>), grid, dim3(64 * kRowsPerBlock), 0, st, m);
  return hipGetLastError();
}

}  // namespace

hipError_t scratch_address(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    // With this device current: its own copy of the array.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = (float*)p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_merge(Dt dt, const MergeParams& m, hipStream_t stream) {
  if ((int64_t)m.B * m.Hq * m.Sq == 0) return hipSuccess;
  return dt == Dt::BF16 ? launch_merge_t<BF16>(m, stream) : launch_merge_t<F16>(m, stream);
}

}  // namespace fa
