// Grouped expert GEMMs (gfx950): launchers for the bf16 and FP8 E4M3 experts.
//
// Sources: [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合 (SwiGLU experts,
// d_ff 2560); [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" §BF16 MoE Kernel Optimization
// (separate decode and prefill tilings; gate/up and activation rounded to bf16; FP32 routing weight
// applied to the down output before rounding) and §BF16, NVFP4 and FP8 Model Support (dynamic FP8).
//
// Operand layout: every operand row runs along the contracted dimension (x rows along H, weight rows
// along H or F), so a lane's consecutive bytes of one row are exactly its MFMA fragment for the
// token operand (A) and the weight operand (B) alike; D holds rows 4*(l/16)+i, column l % 16.
// Row blocks come from moe_align: (expert, first sorted row, rows). Grids are sized by an upper
// bound on the block count; blocks past the device-side count exit at once (no host readback).
//   small blocks (<= 16 rows, decode): grouped_small_kernel, weights streamed into registers;
//     grouped_small_ks_kernel (K split across the waves of a workgroup) where the shape allows.
//   large blocks (320 rows; prefill): grouped_pipe_kernel, LDS rings fed by
//     direct loads.
#include <algorithm>

#include "device_common.h"
#include "gemm_pipe.h"
#include "gemm_small.h"

namespace beam {

static_assert(kSmallBM == kSmallBlockRows, "block rows of the streaming GEMMs");
static_assert(PipeCfg<false>::BM == kPipeBlockRows && PipeCfg<true>::BM == kPipeBlockRows,
              "block rows of the tiled GEMMs");

template <bool GATE_UP, bool FP8>
static void launch_one(const void* a, const void* w, void* out,
                       const float* a_scale, const float* w_scale, const AlignTables& at,
                       int Kd, int Nout, int topk, int64_t max_blocks, bool small,
                       hipStream_t st, int ksplit = 1) {
  const auto* A = reinterpret_cast<const unsigned char*>(a);
  const auto* W = reinterpret_cast<const unsigned char*>(w);
  if (small) {
    // K split across the 4 waves of 16-column (down: 32-column) workgroups: 4x the workgroups of
    // the column-tiled grid (which leaves most CUs idle at a handful of tokens) and two batches in
    // flight per wave; faster at every decode size measured (T = 1 .. 64). The column-tiled
    // kernel covers the shapes whose rows do not split into whole batches.
    const int64_t row_bytes = (int64_t)Kd * (FP8 ? 1 : 2);
    constexpr int64_t BB = KsBatch<FP8>::kBytes;
    const dim3 grid(Nout / (GATE_UP ? 16 : 32), (unsigned)max_blocks);
    if ((row_bytes / 4) % BB == 0) {
      hipLaunchKernelGGL((grouped_small_ks_kernel<GATE_UP, FP8, 4>), grid, dim3(256), 0, st, A, W,
                         out, at, Kd, Nout, topk, a_scale, w_scale);
    } else {
      hipLaunchKernelGGL((grouped_small_kernel<GATE_UP, FP8>),
                         dim3(Nout / kSmallCols, (unsigned)max_blocks), dim3(256), 0, st, A, W,
                         out, at, Kd, Nout, topk, a_scale, w_scale);
    }
  } else {
    const int n_ctiles = GATE_UP ? Nout / 128 : Nout / 256;
    const int64_t wgs = 8 * ceil_div(max_blocks * n_ctiles * ksplit, 8);
    hipLaunchKernelGGL((grouped_pipe_kernel<GATE_UP, FP8>), dim3((unsigned)wgs),
                       dim3(64 * PipeCfg<FP8>::WAVES), 0, st, A, W, out, at, Kd, Nout, topk,
                       n_ctiles, a_scale, w_scale, ksplit);
  }
}

hipError_t launch_gate_up(const void* x, const void* w_gu, uint16_t* hbuf, const float* x_scale,
                          const float* w_scale, bool fp8, const AlignTables& at, const Shape& s,
                          int64_t max_blocks, bool small, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (fp8)
    launch_one<true, true>(x, w_gu, hbuf, x_scale, w_scale, at, s.H, s.F, s.K,
                           max_blocks, small, st);
  else
    launch_one<true, false>(x, w_gu, hbuf, nullptr, nullptr, at, s.H, s.F, s.K,
                            max_blocks, small, st);
  return hipGetLastError();
}

hipError_t launch_down(const void* h, const void* w_dn, const float* h_scale, const float* w_scale,
                       bool fp8, float* ybuf, const AlignTables& at, const Shape& s,
                       int64_t max_blocks, bool small, hipStream_t st, int ksplit) {
  if (s.T == 0) return hipSuccess;
  if (ksplit != 1 && (small || (s.F * (fp8 ? 1 : 2) / kPRowBytes) % ksplit != 0))
    return hipErrorInvalidValue;
  if (fp8)
    launch_one<false, true>(h, w_dn, ybuf, h_scale, w_scale, at, s.F, s.H, s.K,
                            max_blocks, small, st, ksplit);
  else
    launch_one<false, false>(h, w_dn, ybuf, nullptr, nullptr, at, s.F, s.H, s.K,
                             max_blocks, small, st, ksplit);
  return hipGetLastError();
}


}  // namespace beam
