// Device-side helpers of the Beam MoE kernels (gfx950): vector types, bf16 rounding, SiLU.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 -------------------------------------------------------------------------------------
// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_round(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}

// SiLU in fp32 with the full-precision exponential and an IEEE division.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

}  // namespace beam
