// Device-side building blocks shared by the gfx950 attention kernels:
// MFMA operand types, 16-bit packing, cross-half wavefront reductions and LDS
// address-space helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// 16-bit element traits. An MFMA operand is 8 elements (one u32x4) per lane;
// v_mfma_f32_32x32x16_{f16,bf16}: lane l holds A[m = l%32][k = 8*(l/32) + e]
// and B[k = 8*(l/32) + e][n = l%32]; the 16 fp32 results sit at
// C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32], i = 0..15.
struct F16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even of two floats into one packed dword (v_cvt_pk_f16_f32).
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  // acc + the two packed values (v_dot2c_f32_f16 against (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
  }
  // acc + a.lo b.lo + a.hi b.hi in fp32 (v_dot2_f32_f16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
  // The two packed values as floats (exact).
  static __device__ __forceinline__ f32x2 unpack2(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
};

struct BF16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even of two floats into one packed dword (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // acc + the two packed values (v_dot2c_f32_bf16 against (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t packed, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
  }
  // acc + a.lo b.lo + a.hi b.hi in fp32 (v_dot2_f32_bf16).
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
  }
  // The two packed values as floats (exact: a bf16 is the upper half of a float).
  static __device__ __forceinline__ f32x2 unpack2(uint32_t w) {
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  }
};

// Reductions between lane l and lane l ^ 32 (the two halves of a wave hold
// the two interleaved key halves of one query column). v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both operands = x, element 0 / 1 hold (own, partner) on the
// lower half and (partner, own) on the upper half.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(a, b, c) in one instruction. The operands are never NaN here (finite
// scores or -inf), so the IEEE quieting that fmaxf chains otherwise pay for
// with extra canonicalising instructions is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLn2 = 0.69314718055994531f;

// LDS pointer from a byte address. The mask (LDS is below 256 KB) tells the
// compiler the address is non-negative, which lets it fold constant offsets
// into the instructions' immediate offset field.
__device__ __forceinline__ const lds_u16* lds_ptr(uint32_t byte_addr) {
  return (const lds_u16*)(size_t)(byte_addr & 0x3FFFFu);
}

// Transposing LDS read (ds_read_b64_tr_b16) from an LDS pointer.
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_u16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// every lane reads 4 consecutive 16-bit elements at its own address; result
// element j of lane i is element (i % 4) of what lane 4*j + i/4 of the same
// group read.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u16*)lds_ptr));
  return __builtin_bit_cast(u32x2, r);
}

}  // namespace fa
