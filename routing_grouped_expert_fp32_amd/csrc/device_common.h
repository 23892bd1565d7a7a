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

// ---- direct-to-LDS loads and wait counts ------------------------------------------------------
// cache-policy operand of the direct loads: non-temporal, for weight streams read once (they
// should not push reused data out of L2)
constexpr int kCachePolicyNT = 2;

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte load per lane from the raw buffer [base, base + bytes) straight into LDS at dst + 16 *
// lane: lane offset voff, wave-uniform offset soff; lanes outside the range read zero. Buffer
// loads rather than global ones because the compiler then waits for LDS reads by count
// (lgkmcnt(n)) instead of draining them all before every MFMA group.
template <int kAux>
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t bytes, uint32_t voff,
                                                  uint32_t soff, lds_void_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      // descriptor word 3: 32-bit data format (untyped loads still need a valid one)
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000),
      dst, 16, voff, soff, 0, kAux);
}

// 16-byte load per lane from the raw buffer [base, base + bytes) into registers (offsets as
// above); lanes outside the range read zero without a memory access.
template <int kAux>
__device__ __forceinline__ u32x4 buffer_load16(const void* base, uint32_t bytes, uint32_t voff,
                                               uint32_t soff) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                   0x00020000),
                 voff, soff, kAux));
}

// s_waitcnt immediates (gfx9 encoding): at most n vector-memory ops outstanding; no LDS op
// outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);

}  // namespace beam
