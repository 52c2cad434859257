// Internal helpers shared by the HIP sources of libtpgemm (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// bf16 <-> fp32 on raw bits. Rounding is to nearest, ties to even; NaN stays
// a quiet NaN.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two floats to two bf16 in one word (lo in bits 0-15): the gfx950 packed
// conversion v_cvt_pk_bf16_f32. Checked on MI355X against the integer
// rounding below over all 2^32 float bit patterns: identical for every
// non-NaN input (denormals included), and every NaN stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The same rounding in integer arithmetic (one value; NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// logistic(t) = 1 / (1 + e^-t) with the hardware reciprocal (v_rcp_f32, about
// 1 ulp) in place of the correctly rounded division, which takes about ten
// instructions; e^-t -> inf gives 0 and e^-t -> 0 gives 1.
__device__ __forceinline__ float sigmoid_f32(float t) { return __builtin_amdgcn_rcpf(1.0f + __expf(-t)); }

// silu(t) = t * logistic(t)
__device__ __forceinline__ float silu_f32(float t) { return t * sigmoid_f32(t); }

}  // namespace tpg
