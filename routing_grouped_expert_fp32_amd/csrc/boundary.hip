// Sublayer boundary after the MoE (gfx950): output RMSNorm, depth-scaled residual add and the next
// sublayer's input RMSNorm in one pass, optionally fused with the top-k combine.
//
// Sources: [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" §MoE and residual stream (every
// sublayer has an RMSNorm before and after it; the n-th residual add is h <- sqrt((n-1)/n) h + x/sqrt(n))
// and §Agent-driven optimization items 1 and 3 (post-norm, scaled residual add and next pre-norm fused,
// FP32 math with BF16 rounding points; after the MoE the same kernel combines the top-8 outputs);
// [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" §Sandwich Normalization and Depth-Scaled
// Residuals (both scaled operands are rounded to the activation dtype before the addition);
// [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §残差流.
//
// Per token t (FP32 arithmetic, bf16 rounding points):
//   y  = sublayer output (with slots: sum over k, in k order, of Y[t*K+k]);  u = bf16(y)
//   p  = bf16(u * r1 * gamma_post),  r1 = 1 / sqrt(mean(u^2) + eps)
//   h' = bf16(bf16(alpha * h) + bf16(beta * p)),  alpha = sqrt((n-1)/n), beta = 1/sqrt(n)
//   x' = bf16(h' * r2 * gamma_next),  r2 = 1 / sqrt(mean(h'^2) + eps)
// One workgroup of 256 threads per token; each thread keeps its chunks of 4 elements in registers
// between the two reductions. Sums of squares: per-thread partials, a fixed xor butterfly per wave,
// then the four wave sums in wave order (deterministic).
#include <type_traits>

#include "device_common.h"

namespace beam {

constexpr int kBndThreads = 256;
constexpr int kBndMaxChunks = 16;   // hidden <= 16 * 4 * 256 = 16384

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // red is reused by the second reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ float bf16r(float v) { return bf16_round(v); }

// MAXCH: 4-float chunks per thread the registers hold (hidden <= MAXCH * 1024); MAXK: slots read
// per chunk (top-k <= MAXK)
template <bool SLOTS, int MAXCH, int MAXK>
__global__ __launch_bounds__(kBndThreads) void boundary_kernel(
    const float* __restrict__ Y, int K, const int32_t* __restrict__ ids, int e_begin, int e_end,
    const void* __restrict__ y, int y_bf16, const uint16_t* h, const float* __restrict__ gp,
    const float* __restrict__ gn, uint16_t* h_out, uint16_t* __restrict__ x_next, int H,
    float alpha, float beta, float eps) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int nch = H / 4;
  // slots of this token that contribute (all K, or those routed into [e_begin, e_end))
  uint32_t slots = 0;
  if constexpr (SLOTS) {
    for (int k = 0; k < K; ++k) {
      const bool in = !ids || (ids[t * K + k] >= e_begin && ids[t * K + k] < e_end);
      slots |= (in ? 1u : 0u) << k;
    }
  }
  floatx4 u[MAXCH];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int ch = threadIdx.x + kBndThreads * j;
    u[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (ch >= nch) continue;
    const int c = 4 * ch;
    floatx4 v;
    if constexpr (SLOTS) {
      // all of the chunk's slot reads issued together (read once: non-temporal), then summed in
      // k order starting from the first contributing slot
      const float* yp = Y + t * K * H + c;
      floatx4 yk[MAXK];
#pragma unroll
      for (int k = 0; k < MAXK; ++k)
        if ((slots >> k) & 1u)
          yk[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(yp + (int64_t)k * H));
      v = floatx4{0.f, 0.f, 0.f, 0.f};
      bool first = true;
#pragma unroll
      for (int k = 0; k < MAXK; ++k) {
        if (!((slots >> k) & 1u)) continue;
        v = first ? yk[k] : v + yk[k];
        first = false;
      }
    } else if (y_bf16) {
      const u32x2 p = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(y) +
                                                      t * H + c);
      v = floatx4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
    } else {
      v = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(y) + t * H + c);
    }
    u[j] = floatx4{bf16r(v.x), bf16r(v.y), bf16r(v.z), bf16r(v.w)};
    ss += u[j].x * u[j].x + u[j].y * u[j].y + u[j].z * u[j].z + u[j].w * u[j].w;
  }
  const float r1 = 1.0f / sqrtf(block_sum(ss, red) / (float)H + eps);
  float ss2 = 0.f;
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int ch = threadIdx.x + kBndThreads * j;
    if (ch >= nch) continue;
    const int c = 4 * ch;
    const u32x2 hp = *reinterpret_cast<const u32x2*>(h + t * H + c);
    const float hv[4] = {bf16_lo(hp.x), bf16_hi(hp.x), bf16_lo(hp.y), bf16_hi(hp.y)};
    const floatx4 g = *reinterpret_cast<const floatx4*>(gp + c);
    const float uv[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
    const float gv[4] = {g.x, g.y, g.z, g.w};
    floatx4 hn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = bf16r(uv[i] * r1 * gv[i]);
      const float a = bf16r(alpha * hv[i]);
      const float b = bf16r(beta * p);
      hn[i] = bf16r(a + b);
    }
    u[j] = hn;   // h' stays in registers for the second norm
    ss2 += hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
    u32x2 o;
    o.x = f32_to_bf16_bits(hn.x) | (f32_to_bf16_bits(hn.y) << 16);
    o.y = f32_to_bf16_bits(hn.z) | (f32_to_bf16_bits(hn.w) << 16);
    *reinterpret_cast<u32x2*>(h_out + t * H + c) = o;
  }
  const float r2 = 1.0f / sqrtf(block_sum(ss2, red) / (float)H + eps);
#pragma unroll
  for (int j = 0; j < MAXCH; ++j) {
    const int ch = threadIdx.x + kBndThreads * j;
    if (ch >= nch) continue;
    const int c = 4 * ch;
    const floatx4 g = *reinterpret_cast<const floatx4*>(gn + c);
    const floatx4 xn = floatx4{u[j].x * r2 * g.x, u[j].y * r2 * g.y, u[j].z * r2 * g.z,
                               u[j].w * r2 * g.w};
    u32x2 o;
    o.x = f32_to_bf16_bits(xn.x) | (f32_to_bf16_bits(xn.y) << 16);
    o.y = f32_to_bf16_bits(xn.z) | (f32_to_bf16_bits(xn.w) << 16);
    *reinterpret_cast<u32x2*>(x_next + t * H + c) = o;
  }
}

static_assert(kBndMaxChunks * 4 * kBndThreads == kBoundaryMaxHidden, "boundary row width");

hipError_t launch_boundary(const BoundaryArgs& b, const float* Y, int K, const int32_t* ids,
                           int e_begin, int e_end, const void* y, bool y_bf16, int64_t T, int H,
                           hipStream_t st) {
  if (T == 0) return hipSuccess;
  // registers sized to the hidden size: chunks per thread 4 / 8 / 16 (slot reads always sized for
  // 16: an 8-slot instantiation lets the compiler hoist every chunk's reads at once, 250 registers
  // and one wave per SIMD, measured 3.8x slower)
  const int nch = ceil_div(H / 4, kBndThreads);
  auto go = [&](auto slots_tag, auto ch_tag, auto k_tag) {
    constexpr bool S = decltype(slots_tag)::value;
    constexpr int CH = decltype(ch_tag)::value, MK = decltype(k_tag)::value;
    if constexpr (S)
      hipLaunchKernelGGL((boundary_kernel<true, CH, MK>), dim3((unsigned)T), dim3(kBndThreads), 0,
                         st, Y, K, ids, e_begin, e_end, nullptr, 0, b.h, b.gamma_post,
                         b.gamma_next, b.h_out, b.x_next, H, b.alpha, b.beta, b.eps);
    else
      hipLaunchKernelGGL((boundary_kernel<false, CH, MK>), dim3((unsigned)T), dim3(kBndThreads),
                         0, st, nullptr, 0, nullptr, 0, 0, y, y_bf16 ? 1 : 0, b.h, b.gamma_post,
                         b.gamma_next, b.h_out, b.x_next, H, b.alpha, b.beta, b.eps);
  };
  using T4 = std::integral_constant<int, 4>;
  using T8 = std::integral_constant<int, 8>;
  using T16 = std::integral_constant<int, 16>;
  auto by_chunks = [&](auto slots_tag, auto k_tag) {
    if (nch <= 4)
      go(slots_tag, T4{}, k_tag);
    else if (nch <= 8)
      go(slots_tag, T8{}, k_tag);
    else
      go(slots_tag, T16{}, k_tag);
  };
  if (Y)
    by_chunks(std::true_type{}, T16{});
  else
    by_chunks(std::false_type{}, T16{});
  return hipGetLastError();
}

}  // namespace beam
