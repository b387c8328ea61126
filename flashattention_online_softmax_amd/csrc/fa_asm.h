// Inline-assembly building blocks of the gfx950 kernels that are compiled
// into the run-time loaded code object: LDS-DMA copies, vector-memory and
// barrier waits, and MFMAs whose accumulator register file (VGPR or AGPR) is
// chosen here rather than by the compiler, with the wait states the compiler
// cannot see through the assembly.
#pragma once

#include <stdint.h>

#include "fa_device.h"

namespace fa {

// A pointer whose value is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i fills LDS bytes [lds_addr + 16 i, +16)
// from gbase + voff. Issued through inline assembly so that the compiler does
// not hold later LDS reads of other buffers behind it; the kernel itself
// waits for these copies (s_waitcnt vmcnt) before the barrier that publishes
// their data. gbase and lds_addr are the same in every lane of the wave (they
// are moved to scalar registers here, a no-op when they already are).
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(gbase))
      : "memory", "m0");
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (gfx9 layout: base, stride 0, size in bytes, 32-bit data
// format) over [base, base + bytes). Buffer loads at offsets at or past
// `bytes` return zeros instead of touching memory.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = (int32_t)__builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// Like lds_copy16, through a buffer resource (buffer_load_dwordx4 ... lds):
// lane i fills LDS bytes [lds_addr + 16 i, +16) from byte offset voff of the
// buffer (zeros past its end). rsrc and lds_addr are wave-uniform.
__device__ __forceinline__ void lds_gather16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
      : "memory", "m0");
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

// MFMA issued through inline assembly so that this code, not the compiler,
// picks the register file of each accumulator: score accumulators live in
// VGPRs (the softmax reads them), output accumulators in AGPRs (only MFMAs
// and the rare rescale touch them). Independent VALU instructions of the same
// wave keep issuing while an MFMA runs.
// Hazards the compiler cannot see through the asm are covered explicitly:
// VALU accesses to an MFMA result wait mfma_wait_v / mfma_wait_a first, and
// an MFMA reading accumulators that VALU code wrote waits acc_written first.
template <class T>
struct Mma;
template <>
struct Mma<BF16> {
  static __device__ __forceinline__ void v0(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void v(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void a(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
  // VGPR accumulator, B operand held in AGPRs. The B operand is declared
  // read-write (the instruction does not change it) so that the compiler
  // keeps it in AGPRs instead of copying it there before every use.
  static __device__ __forceinline__ void v0b(f32x16& d, u32x4 a, u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %1, 0" : "=&v"(d), "+a"(b) : "v"(a));
  }
  static __device__ __forceinline__ void vb(f32x16& d, u32x4 a, u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %1, %0" : "+v"(d), "+a"(b) : "v"(a));
  }
};
template <>
struct Mma<F16> {
  static __device__ __forceinline__ void v0(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void v(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void a(f32x16& d, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
  // VGPR accumulator, B operand held in AGPRs. The B operand is declared
  // read-write (the instruction does not change it) so that the compiler
  // keeps it in AGPRs instead of copying it there before every use.
  static __device__ __forceinline__ void v0b(f32x16& d, u32x4 a, u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %2, %1, 0" : "=&v"(d), "+a"(b) : "v"(a));
  }
  static __device__ __forceinline__ void vb(f32x16& d, u32x4 a, u32x4& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %2, %1, %0" : "+v"(d), "+a"(b) : "v"(a));
  }
};

// Wait states between the last 32x32x16 MFMA writing a register and a VALU
// instruction touching it (more than the 8-pass MFMA needs). The registers
// are operands of the wait so that the compiler places every access to them
// after it.
template <int N>
__device__ __forceinline__ void mfma_wait_v(f32x16 (&a)[N]) {
  static_assert(N >= 1 && N <= 4, "tiles");
  if constexpr (N == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  else if constexpr (N == 3)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]));
  else if constexpr (N == 2)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a[0]), "+v"(a[1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a[0]));
}
template <int N>
__device__ __forceinline__ void mfma_wait_a(f32x16 (&a)[N]) {
  static_assert(N == 2 || N == 4, "d tiles");
  if constexpr (N == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]));
}
// Wait states between VALU writes of VGPR accumulators and the next MFMA
// reading them; the writes are placed before it.
template <int N>
__device__ __forceinline__ void vacc_written(f32x16 (&a)[N]) {
  static_assert(N == 2 || N == 4, "d tiles");
  if constexpr (N == 4)
    asm volatile("s_nop 4" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  else
    asm volatile("s_nop 4" : "+v"(a[0]), "+v"(a[1]));
}
// Wait states between VALU writes of accumulator registers and the next
// MFMA reading them; the writes are placed before it.
template <int N>
__device__ __forceinline__ void acc_written(f32x16 (&a)[N]) {
  if constexpr (N == 4)
    asm volatile("s_nop 4" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
  else
    asm volatile("s_nop 4" : "+a"(a[0]), "+a"(a[1]));
}

}  // namespace fa
