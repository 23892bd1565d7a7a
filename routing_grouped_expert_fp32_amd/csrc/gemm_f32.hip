// FP32 experts (no rounding point anywhere), for FP32 activations and weights (gfx950).
//
// Same block structure as the bf16 path (rows grouped per expert by moe_align into blocks of at most
// 16 rows). Each wave computes one 16-row x 16-column tile on the FP32 matrix cores
// (v_mfma_f32_16x16x4_f32): lane (r, g) = (lane % 16, lane / 16) loads four consecutive K values of
// row r of each operand per 16-deep chunk, and MFMA step c consumes component c, so step c sums the
// K offsets {c, 4 + c, 8 + c, 12 + c} - the same permutation on both operands, hence the same
// products, accumulated in FP32. Four waves cover 64 output columns.
// SwiGLU without biases: [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合.
#include "device_common.h"

namespace beam {

// Tile of A rows (this lane's row: a) times B rows (this lane's column: b) over K; lane holds
// D[4 g + q][r], q = 0..3.
__device__ __forceinline__ floatx4 mfma_tile_f32(const float* __restrict__ a,
                                                 const float* __restrict__ b, int K, int g) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; k += 16) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(a + k + 4 * g);
    const floatx4 y = *reinterpret_cast<const floatx4*>(b + k + 4 * g);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, y.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, y.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, y.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, y.w, acc, 0, 0, 0);
  }
  return acc;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          float* __restrict__ hbuf, AlignTables at,
                                                          int H, int F, int topk) {
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;   // block-uniform
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int col = blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + r;   // this lane's output column
  const int rr = r < rows ? r : 0;                                 // padding rows re-read row 0
  const float* xr = x + (int64_t)(at.sorted_slot[row0 + rr] / topk) * H;
  const floatx4 gv = mfma_tile_f32(xr, W + ((int64_t)e * 2 * F + col) * H, H, g);
  const floatx4 uv = mfma_tile_f32(xr, W + ((int64_t)e * 2 * F + F + col) * H, H, g);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * g + q;
    if (row < rows) hbuf[(int64_t)(row0 + row) * F + col] = silu_f32(gv[q]) * uv[q];
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
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int col = blockIdx.x * 64 + (threadIdx.x >> 6) * 16 + r;
  const int rr = r < rows ? r : 0;
  const floatx4 y = mfma_tile_f32(hbuf + (int64_t)(row0 + rr) * F,
                                  W + ((int64_t)e * H + col) * F, F, g);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * g + q;
    if (row < rows) {
      const int slot = at.sorted_slot[row0 + row];
      ybuf[(int64_t)slot * H + col] = topk_w[slot] * y[q];
    }
  }
}

hipError_t launch_gate_up_f32(const float* x, const float* w_gu, float* hbuf,
                              const AlignTables& at, const Shape& s, int64_t max_blocks,
                              hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  static_assert(kSmallBlockRows == 16, "one 16-row MFMA tile per block");
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
