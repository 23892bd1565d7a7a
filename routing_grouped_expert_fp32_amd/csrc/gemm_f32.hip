// FP32 experts (no rounding point anywhere), for FP32 activations and weights (gfx950).
//
// Same block structure as the bf16 path (rows grouped per expert by moe_align), one thread per
// (row, output column), FP32 fused multiply-adds along the contracted dimension.
// SwiGLU without biases: [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合.
#include "device_common.h"

namespace beam {

__device__ __forceinline__ float dot_f32(const float* __restrict__ a, const float* __restrict__ b,
                                         int n) {
  float s = 0.f;
  for (int k = 0; k < n; k += 4) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(a + k);
    const floatx4 y = *reinterpret_cast<const floatx4*>(b + k);
    s = fmaf(x.x, y.x, s);
    s = fmaf(x.y, y.y, s);
    s = fmaf(x.z, y.z, s);
    s = fmaf(x.w, y.w, s);
  }
  return s;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          float* __restrict__ hbuf, AlignTables at,
                                                          int H, int F, int topk) {
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const float* wg = W + ((int64_t)e * 2 * F + col) * H;
  const float* wu = W + ((int64_t)e * 2 * F + F + col) * H;
  for (int rr = threadIdx.x >> 6; rr < rows; rr += 4) {
    const float* xr = x + (int64_t)(at.sorted_slot[row0 + rr] / topk) * H;
    const float gv = dot_f32(xr, wg, H), uv = dot_f32(xr, wu, H);
    hbuf[(int64_t)(row0 + rr) * F + col] = silu_f32(gv) * uv;
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ hbuf,
                                                       const float* __restrict__ W,
                                                       const float* __restrict__ topk_w,
                                                       float* __restrict__ ybuf, AlignTables at,
                                                       int H, int F) {
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const float* wd = W + ((int64_t)e * H + col) * F;
  for (int rr = threadIdx.x >> 6; rr < rows; rr += 4) {
    const int slot = at.sorted_slot[row0 + rr];
    const float y = dot_f32(hbuf + (int64_t)(row0 + rr) * F, wd, F);
    ybuf[(int64_t)slot * H + col] = topk_w[slot] * y;
  }
}

hipError_t launch_gate_up_f32(const float* x, const float* w_gu, float* hbuf,
                              const AlignTables& at, const Shape& s, int64_t max_blocks,
                              hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_up_f32_kernel, dim3(s.F / 64, (unsigned)max_blocks), dim3(256), 0, st,
                     x, w_gu, hbuf, at, s.H, s.F, s.K);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* hbuf, const float* w_dn, const float* topk_w, float* ybuf,
                           const AlignTables& at, const Shape& s, int64_t max_blocks,
                           hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  hipLaunchKernelGGL(down_f32_kernel, dim3(s.H / 64, (unsigned)max_blocks), dim3(256), 0, st,
                     hbuf, w_dn, topk_w, ybuf, at, s.H, s.F);
  return hipGetLastError();
}

}  // namespace beam
