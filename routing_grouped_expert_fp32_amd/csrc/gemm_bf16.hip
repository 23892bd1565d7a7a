// Grouped expert GEMMs on bf16 MFMA (gfx950, v_mfma_f32_16x16x32_bf16), with fused epilogues.
//
// Sources: [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合 (SwiGLU experts,
// d_ff 2560); [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" §BF16 MoE Kernel Optimization
// (separate decode and prefill tilings; gate/up and activation rounded to bf16; FP32 routing weight
// applied to the down output before rounding).
//
// Operand layout: every operand row runs along the contracted dimension (x rows along H, weight rows
// along H or F), so a lane's 8 consecutive bf16 (16 bytes) of one row are exactly its MFMA fragment:
// lane l supplies row (l % 16) and K slice [8*(l/16), 8*(l/16)+8) of a 32-deep step, for the token
// operand (A) and the weight operand (B) alike. D holds rows 4*(l/16)+i, column l % 16.
//
// gate/up: for the rows of one block (one expert e), g = x . Wg[e]^T and u = x . Wu[e]^T with the
// gate and up columns of the same h index in the same lane, so the epilogue
//   h = bf16( silu(bf16(g)) * bf16(u) )   (fp32 arithmetic)
// runs in registers and writes h (bf16) in sorted-row order.
// down: y = h . Wd[e]^T; the epilogue writes Y[slot] = topk_w[slot] * y in fp32 (slot = t*K+k).
//
// Row blocks come from moe_align: (expert, first sorted row, rows). Grids are sized by an upper
// bound on the block count; blocks past the device-side count exit at once (no host readback).
#include "common.h"
#include "gemm_pipe.h"

namespace beam {

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// Small blocks (<= 16 rows): weight streaming. WG = 4 waves x 16 output columns; each lane streams
// its weight row(s) straight from HBM into MFMA registers, kSmallU 32-deep steps per batch.
constexpr int kSmallBM = 16;
constexpr int kSmallCols = 64;
constexpr int kSmallU = 8;

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_small_kernel(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ W,
                                                            const float* __restrict__ topk_w,
                                                            void* __restrict__ out, AlignTables at,
                                                            int Kd, int Nout, int topk) {
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * kSmallCols + wave * 16;

  const uint16_t* ap = nullptr;
  if (r < rows) {
    if constexpr (GATE_UP)
      ap = A + (int64_t)(at.sorted_slot[row0 + r] / topk) * Kd;
    else
      ap = A + (int64_t)(row0 + r) * Kd;
  }
  const uint16_t* bp0;
  const uint16_t* bp1 = nullptr;
  if constexpr (GATE_UP) {
    bp0 = W + ((int64_t)e * 2 * Nout + c0 + r) * Kd;
    bp1 = W + ((int64_t)e * 2 * Nout + Nout + c0 + r) * Kd;
  } else {
    bp0 = W + ((int64_t)e * Nout + c0 + r) * Kd;
  }
  const int koff = g * 8;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 zero = {};
  for (int k = 0; k < Kd; k += 32 * kSmallU) {
    bf16x8 a[kSmallU], w0[kSmallU], w1[kSmallU];
#pragma unroll
    for (int u = 0; u < kSmallU; ++u) {
      w0[u] = ld16(bp0 + k + 32 * u + koff);
      if constexpr (GATE_UP) w1[u] = ld16(bp1 + k + 32 * u + koff);
    }
#pragma unroll
    for (int u = 0; u < kSmallU; ++u) a[u] = ap ? ld16(ap + k + 32 * u + koff) : zero;
#pragma unroll
    for (int u = 0; u < kSmallU; ++u) {
      acc0 = mfma16(a[u], w0[u], acc0);
      if constexpr (GATE_UP) acc1 = mfma16(a[u], w1[u], acc1);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    if (row >= rows) continue;
    if constexpr (GATE_UP) {
      const float h = silu_f32(bf16_round(acc0[i])) * bf16_round(acc1[i]);
      reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + c0 + r] =
          (uint16_t)f32_to_bf16_bits(h);
    } else {
      const int slot = at.sorted_slot[row0 + row];
      reinterpret_cast<float*>(out)[(int64_t)slot * Nout + c0 + r] = topk_w[slot] * acc0[i];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Large blocks (<= 128 rows): LDS-tiled, double-buffered. WG tile 128 rows x 128 weight columns
// (gate/up: 64 gate + the 64 matching up columns), K tile 64; 4 waves as 2 x 2, wave tile
// 64 rows x 64 columns = 4 x 4 MFMA tiles. Row sub-tiles entirely past the block's rows skip
// their MFMAs (wave-uniform test).
constexpr int kTBM = 128;
constexpr int kTBN = 128;
constexpr int kTBK = 64;
constexpr int kTLd = kTBK + 8;   // padded LDS row (144 B) to spread rows over banks

template <bool GATE_UP>
__global__ __launch_bounds__(256, 2) void grouped_tiled_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W,
                                                               const float* __restrict__ topk_w,
                                                               void* __restrict__ out,
                                                               AlignTables at, int Kd, int Nout,
                                                               int topk) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTBM * kTLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTBN * kTLd];
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;
  const int j = blockIdx.x;

  // global -> LDS mapping: thread covers rows lrow + 32i, 8 bf16 at column lk
  const int lrow = tid >> 3, lk = (tid & 7) * 8;
  const uint16_t* ap[4];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = lrow + 32 * i;
    ap[i] = nullptr;
    if (rr < rows) {
      if constexpr (GATE_UP)
        ap[i] = A + (int64_t)(at.sorted_slot[row0 + rr] / topk) * Kd + lk;
      else
        ap[i] = A + (int64_t)(row0 + rr) * Kd + lk;
    }
    if constexpr (GATE_UP) {
      const int wrow = rr < 64 ? 64 * j + rr : Nout + 64 * j + (rr - 64);
      bp[i] = W + ((int64_t)e * 2 * Nout + wrow) * Kd + lk;
    } else {
      bp[i] = W + ((int64_t)e * Nout + kTBN * j + rr) * Kd + lk;
    }
  }
  u32x4 ra[4], rb[4];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ap[i] ? *reinterpret_cast<const u32x4*>(ap[i] + k) : zero4;
      rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][(lrow + 32 * i) * kTLd + lk]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][(lrow + 32 * i) * kTLd + lk]) = rb[i];
    }
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  const int nk = Kd / kTBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kTBK);
#pragma unroll
    for (int ks = 0; ks < kTBK / 32; ++ks) {
      bf16x8 af[4], bw[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        af[ms] = *reinterpret_cast<const bf16x8*>(
            &As[cur][(wm * 64 + ms * 16 + r) * kTLd + ks * 32 + g * 8]);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        int brow;
        if constexpr (GATE_UP)
          brow = ns < 2 ? wn * 32 + ns * 16 + r : 64 + wn * 32 + (ns - 2) * 16 + r;
        else
          brow = wn * 64 + ns * 16 + r;
        bw[ns] = *reinterpret_cast<const bf16x8*>(&Bs[cur][brow * kTLd + ks * 32 + g * 8]);
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (wm * 64 + ms * 16 >= rows) continue;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = mfma16(af[ms], bw[ns], acc[ms][ns]);
      }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + ms * 16 + 4 * g + i;
      if (row >= rows) continue;
      if constexpr (GATE_UP) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float h = silu_f32(bf16_round(acc[ms][p][i])) * bf16_round(acc[ms][p + 2][i]);
          const int hcol = 64 * j + wn * 32 + p * 16 + r;
          reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + hcol] =
              (uint16_t)f32_to_bf16_bits(h);
        }
      } else {
        const int slot = at.sorted_slot[row0 + row];
        const float wgt = topk_w[slot];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const int col = kTBN * j + wn * 64 + ns * 16 + r;
          reinterpret_cast<float*>(out)[(int64_t)slot * Nout + col] = wgt * acc[ms][ns][i];
        }
      }
    }
  }
}

int small_block_rows() { return kSmallBM; }
int tiled_block_rows() { return kPBM; }

hipError_t launch_gate_up_bf16(const uint16_t* x, const uint16_t* w_gu, uint16_t* hbuf,
                               const AlignTables& at, const Shape& s, int64_t max_blocks,
                               bool small, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (small) {
    dim3 grid(s.F / kSmallCols, (unsigned)max_blocks);
    hipLaunchKernelGGL((grouped_small_kernel<true>), grid, dim3(256), 0, st, x, w_gu, nullptr,
                       hbuf, at, s.H, s.F, s.K);
  } else {
    const int n_ctiles = s.F / 128;
    const int64_t wgs = 8 * ceil_div(max_blocks * n_ctiles, 8);
    hipLaunchKernelGGL((grouped_pipe_kernel<true>), dim3((unsigned)wgs), dim3(256), 0, st, x,
                       w_gu, nullptr, hbuf, at, s.H, s.F, s.K, n_ctiles);
  }
  return hipGetLastError();
}

hipError_t launch_down_bf16(const uint16_t* hbuf, const uint16_t* w_dn, const float* topk_w,
                            float* ybuf, const AlignTables& at, const Shape& s,
                            int64_t max_blocks, bool small, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (small) {
    dim3 grid(s.H / kSmallCols, (unsigned)max_blocks);
    hipLaunchKernelGGL((grouped_small_kernel<false>), grid, dim3(256), 0, st, hbuf, w_dn, topk_w,
                       ybuf, at, s.F, s.H, s.K);
  } else {
    const int n_ctiles = s.H / 256;
    const int64_t wgs = 8 * ceil_div(max_blocks * n_ctiles, 8);
    hipLaunchKernelGGL((grouped_pipe_kernel<false>), dim3((unsigned)wgs), dim3(256), 0, st, hbuf,
                       w_dn, topk_w, ybuf, at, s.F, s.H, s.K, n_ctiles);
  }
  return hipGetLastError();
}

}  // namespace beam
