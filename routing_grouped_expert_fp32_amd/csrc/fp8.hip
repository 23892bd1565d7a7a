// Dynamic FP8 E4M3 quantisation of activation rows (gfx950).
//
// [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" §Highlights and §BF16, NVFP4 and FP8 Model
// Support (compressed-tensors dynamic FP8 checkpoints); the format is OCP E4M3FN (largest finite
// 448, no infinities), gfx950's native FP8 operand format.
// Per row of bf16 values v (x per token before gate/up, h per sorted row before down):
//   amax = max |v| (exact); scale = amax / 448, inv = 448 / amax (FP32, correctly rounded);
//   code = E4M3(v * inv) rounded to nearest even and saturated to +-448; amax = 0 gives scale 1 and
//   all-zero codes. The encoder is written out in integer arithmetic so the codes do not depend on
//   any hardware conversion mode; the sign of zero follows the input (-0 -> 0x80).
#include <algorithm>

#include "device_common.h"

namespace beam {

__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a < 464.0f)) return sign | 0x7Eu;        // at or past 464 every rounding exceeds 448
  if (a < 0.015625f) {                           // below 2^-6: subnormal grid of step 2^-9
    const uint32_t m = (uint32_t)__float2int_rn(a * 512.0f);   // exact scaling, RNE to integer
    return sign | m;                             // m = 8 is the smallest normal (0x08)
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);              // round the fp32 mantissa to 3 bits, ties to even
  const uint32_t exp = (u >> 23) - 127u + 7u;    // E4M3 biased exponent (>= 1 here)
  const uint32_t man = (u >> 20) & 7u;
  if (exp > 15u || (exp == 15u && man == 7u)) return sign | 0x7Eu;   // rounded past 448
  return sign | (exp << 3) | man;
}

// Four codes packed in a word, by the hardware conversion (round to nearest even, OCP E4M3FN on
// gfx950). The quantisers feed it fp32(v * 448 / amax), whose magnitude is at most 448 plus a
// rounding, where it agrees with e4m3_rne_sat (checked against the oracle's codes bit for bit);
// e4m3_rne_sat stays the encoder of beam_moe_convert, whose inputs can exceed the FP8 range.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// eight bf16 values (one 16-byte load) -> eight codes
__device__ __forceinline__ u32x2 encode8(const u32x4& q, float inv) {
  return u32x2{e4m3x4(bf16_lo(q.x) * inv, bf16_hi(q.x) * inv, bf16_lo(q.y) * inv, bf16_hi(q.y) * inv),
               e4m3x4(bf16_lo(q.z) * inv, bf16_hi(q.z) * inv, bf16_lo(q.w) * inv, bf16_hi(q.w) * inv)};
}

// one workgroup per row; cols % 8 == 0 (8 values = one 16-byte load). n_rows (device, nullable):
// rows at or past *n_rows are not quantised (a routed call's h holds only its local rows).
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t* __restrict__ src,
                                                             int cols, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             const int32_t* __restrict__ n_rows) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  if (n_rows && row >= *n_rows) return;   // whole workgroup
  const uint16_t* p = src + row * cols;
  const int n8 = cols >> 3;
  float amax = 0.f;
  for (int c = threadIdx.x; c < n8; c += 256) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p + 8 * c);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool zero = !(amax > 0.f);
  const float inv = zero ? 0.f : __fdiv_rn(448.0f, amax);
  if (threadIdx.x == 0) scales[row] = zero ? 1.0f : __fdiv_rn(amax, 448.0f);
  for (int c = threadIdx.x; c < n8; c += 256) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p + 8 * c);
    *reinterpret_cast<u32x2*>(codes + row * cols + 8 * c) = zero ? u32x2{0u, 0u} : encode8(q, inv);
  }
}

// Many short rows (the h rows of a prefill batch): one wave per row, four rows per workgroup, the
// row held in registers between the amax and the encode (CH 16-byte pieces per lane, rows of up to
// 512 * CH values), no LDS or barrier; h at T=8192 (65536 rows of 2560) 0.183 -> 0.146 ms. Few or
// long rows (x, decode batches) keep the workgroup per row: fewer waves per row there left the
// GPU underfilled or, with the long x rows in registers, at two waves per SIMD.
template <int CH>
__global__ __launch_bounds__(256) void quant_rows_fp8_wave_kernel(const uint16_t* __restrict__ src,
                                                             int64_t rows, int cols,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             const int32_t* __restrict__ n_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows || (n_rows && row >= *n_rows)) return;   // whole wave; no workgroup barrier below
  const uint16_t* p = src + row * cols;
  const int n8 = cols >> 3;
  auto amax8 = [](const u32x4& q, float m) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
    return m;
  };
  float amax = 0.f;
  u32x4 q[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = lane + 64 * i;
    q[i] = c < n8 ? *reinterpret_cast<const u32x4*>(p + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) amax = amax8(q[i], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const bool zero = !(amax > 0.f);
  const float inv = zero ? 0.f : __fdiv_rn(448.0f, amax);
  if (lane == 0) scales[row] = zero ? 1.0f : __fdiv_rn(amax, 448.0f);
  uint8_t* const o = codes + row * cols;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = lane + 64 * i;
    if (c < n8) *reinterpret_cast<u32x2*>(o + 8 * c) = zero ? u32x2{0u, 0u} : encode8(q[i], inv);
  }
}

// Element conversions with the rounding routines the kernels use: fp32 -> bf16 (round to nearest
// even) or fp32 -> E4M3 (round to nearest even, saturating), four elements per thread.
template <bool TO_FP8>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, int64_t n,
                                                      void* __restrict__ dst) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = i0; i < n; i += stride) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i + u >= n) break;
      const float v = src[i + u];
      if constexpr (TO_FP8)
        reinterpret_cast<uint8_t*>(dst)[i + u] = (uint8_t)e4m3_rne_sat(v);
      else
        reinterpret_cast<uint16_t*>(dst)[i + u] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// One 16x16x128 E4M3 MFMA per tile (the instruction of the FP8 expert GEMMs, unit block scales):
// D = A B^T + C for A [16][128] and B [16][128] codes (each row along K) and C, D [16][16] FP32.
__global__ __launch_bounds__(64) void fp8_dot_tile_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ B,
                                                          const float* __restrict__ C,
                                                          float* __restrict__ D, int64_t n) {
  const int64_t t = blockIdx.x;
  if (t >= n) return;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const uint8_t* a = A + t * 2048 + r * 128 + 32 * g;
  const uint8_t* b = B + t * 2048 + r * 128 + 32 * g;
  const intx4 a0 = *reinterpret_cast<const intx4*>(a), a1 = *reinterpret_cast<const intx4*>(a + 16);
  const intx4 b0 = *reinterpret_cast<const intx4*>(b), b1 = *reinterpret_cast<const intx4*>(b + 16);
  const intx8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const intx8 bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  floatx4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = C[t * 256 + (4 * g + i) * 16 + r];
  const floatx4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
#pragma unroll
  for (int i = 0; i < 4; ++i) D[t * 256 + (4 * g + i) * 16 + r] = d[i];
}

hipError_t launch_fp8_dot_tiles(const uint8_t* A, const uint8_t* B, const float* C, float* D,
                                int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_dot_tile_kernel, dim3((unsigned)n), dim3(64), 0, st, A, B, C, D, n);
  return hipGetLastError();
}

hipError_t launch_convert(const float* src, int64_t n, bool to_fp8, void* dst, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(n, 1024), 65536);
  if (to_fp8)
    hipLaunchKernelGGL(convert_kernel<true>, dim3(grid), dim3(256), 0, st, src, n, dst);
  else
    hipLaunchKernelGGL(convert_kernel<false>, dim3(grid), dim3(256), 0, st, src, n, dst);
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                 float* scales, hipStream_t st, const int32_t* n_rows) {
  if (rows == 0) return hipSuccess;
  const int64_t per_lane = ceil_div((int64_t)cols / 8, 64);   // 16-byte pieces per lane of a wave
  if (rows >= 16384 && per_lane <= 8) {
    const dim3 grid((unsigned)ceil_div(rows, 4));
    if (per_lane <= 5)
      hipLaunchKernelGGL(quant_rows_fp8_wave_kernel<5>, grid, dim3(256), 0, st, src, rows, cols,
                         codes, scales, n_rows);
    else
      hipLaunchKernelGGL(quant_rows_fp8_wave_kernel<8>, grid, dim3(256), 0, st, src, rows, cols,
                         codes, scales, n_rows);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)rows), dim3(256), 0, st, src, cols,
                     codes, scales, n_rows);
  return hipGetLastError();
}

}  // namespace beam
