// Weighted combine with no shared expert (gfx950):
//   out[t] = Y[t*K+0] + Y[t*K+1] + ... + Y[t*K+K-1]   (FP32, fixed k order)
// where Y[slot] already holds topk_w[slot] * expert output (applied by the down GEMM's epilogue).
// [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" §MoE and residual stream (no shared
// expert); [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合 (outputs combined with
// the normalised router weights times 2.5). A bf16 output is the round-to-nearest-even of the FP32 sum.
// With given routes over a range of experts ([S] §Fusion Optimizations: expert IDs and weights in,
// complete outputs back, every expert-parallel rank running its own experts) the sum covers the
// slots routed to the range.
#include "device_common.h"

namespace beam {

// Y is read once: non-temporal loads (measured 17% faster than cached ones at T=8192).
// FILTER: only slots whose id lies in [e_begin, e_end) contribute (a routed call over a range of
// experts; the other slots' Y rows were never written); the sum then starts from +0.
constexpr int kCombineMaxSlots = 16;   // top-k <= 16

template <bool FILTER>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      void* __restrict__ out, int out_bf16,
                                                      int H, int K,
                                                      const int32_t* __restrict__ ids, int e_begin,
                                                      int e_end) {
  const int64_t t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  const float* y = Y + t * K * H + c;
  // contributing slots (all K, or those routed into [e_begin, e_end)); their reads are issued
  // together, then summed in k order
  uint32_t slots = K >= 32 ? ~0u : (1u << K) - 1u;
  if constexpr (FILTER) {
    slots = 0;
    for (int k = 0; k < K; ++k)
      slots |= (ids[t * K + k] >= e_begin && ids[t * K + k] < e_end ? 1u : 0u) << k;
  }
  floatx4 yk[kCombineMaxSlots];
#pragma unroll
  for (int k = 0; k < kCombineMaxSlots; ++k)
    if ((slots >> k) & 1u)
      yk[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(y + (int64_t)k * H));
  floatx4 acc;
  if constexpr (FILTER) {
    acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kCombineMaxSlots; ++k)
      if ((slots >> k) & 1u) acc += yk[k];
  } else {
    acc = yk[0];
#pragma unroll
    for (int k = 1; k < kCombineMaxSlots; ++k)
      if ((slots >> k) & 1u) acc += yk[k];
  }
  if (out_bf16) {
    u32x2 p;
    p.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
    p.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + t * H + c) = p;
  } else {
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(out) + t * H + c) = acc;
  }
}

hipError_t launch_combine(const float* ybuf, void* out, bool out_bf16, const Shape& s,
                          const int32_t* ids, int e_begin, int e_end, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)s.T, (unsigned)ceil_div(s.H, 1024));
  if (ids)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st, ybuf, out, out_bf16 ? 1 : 0,
                       s.H, s.K, ids, e_begin, e_end);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st, ybuf, out, out_bf16 ? 1 : 0,
                       s.H, s.K, ids, e_begin, e_end);
  return hipGetLastError();
}

}  // namespace beam
