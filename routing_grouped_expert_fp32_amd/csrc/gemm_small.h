// Weight-streaming grouped GEMM for small row blocks (<= 16 rows; decode-sized batches), gfx950.
//
// At decode each touched expert carries a handful of rows, so every weight byte is used once or
// twice: the kernel is an HBM stream. WG = 4 waves x 16 output columns; each lane streams its
// weight row(s) straight from HBM into MFMA operand registers (no LDS), 512 bytes of every row per
// batch with all of a batch's loads issued before its MFMAs (a row's last bytes short of a batch go
// one MFMA step at a time). Token rows past the block's rows are
// zero operands and their results are discarded.
//   bf16: v_mfma_f32_16x16x32_bf16, lane = row (l % 16), 16 bytes at K slice 8*(l/16) of each
//         32-deep step; 8 steps per batch.
//   FP8:  16x16x128 f8f6f4 MFMA (E4M3, unit block scales), 32 bytes at K slice 32*(l/16) of each
//         128-deep step; 4 steps per batch.
// Epilogues as in the pipelined kernel: gate/up h = bf16(silu(bf16(g)) * bf16(u)); down
// Y[slot] = topk_w[slot] * y (FP32); FP8 accumulators are dequantised (token/row scale x output-
// channel scale) first.
#pragma once
#include "device_common.h"

namespace beam {

constexpr int kSmallBM = 16;
constexpr int kSmallCols = 64;
constexpr int kSmallBatchBytes = 512;   // bytes of each operand row per batch

template <bool FP8>
struct SmallMath;
template <>
struct SmallMath<false> {
  using frag = bf16x8;
  static constexpr int kStepBytes = 64, kLaneBytes = 16, kElemBytes = 2;
  __device__ static frag load(const unsigned char* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static frag zero() { return frag{}; }
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct SmallMath<true> {
  using frag = intx8;
  static constexpr int kStepBytes = 128, kLaneBytes = 32, kElemBytes = 1;
  __device__ static frag load(const unsigned char* p) {
    const intx4 lo = *reinterpret_cast<const intx4*>(p);
    const intx4 hi = *reinterpret_cast<const intx4*>(p + 16);
    return frag{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  __device__ static frag zero() { return frag{0, 0, 0, 0, 0, 0, 0, 0}; }
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <bool GATE_UP, bool FP8>
__global__ __launch_bounds__(256) void grouped_small_kernel(
    const unsigned char* __restrict__ A, const unsigned char* __restrict__ W,
    void* __restrict__ out, AlignTables at, int Kd, int Nout,
    int topk, const float* __restrict__ a_scale, const float* __restrict__ w_scale) {
  using M = SmallMath<FP8>;
  constexpr int U = kSmallBatchBytes / M::kStepBytes;   // MFMA steps per batch
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * kSmallCols + wave * 16;
  const int64_t row_bytes = (int64_t)Kd * M::kElemBytes;

  const unsigned char* ap = nullptr;
  if (r < rows) {
    if constexpr (GATE_UP)
      ap = A + (int64_t)(at.sorted_slot[row0 + r] / topk) * row_bytes;
    else
      ap = A + (int64_t)(row0 + r) * row_bytes;
  }
  const unsigned char* bp0;
  const unsigned char* bp1 = nullptr;
  if constexpr (GATE_UP) {
    bp0 = W + ((int64_t)e * 2 * Nout + c0 + r) * row_bytes;
    bp1 = W + ((int64_t)e * 2 * Nout + Nout + c0 + r) * row_bytes;
  } else {
    bp0 = W + ((int64_t)e * Nout + c0 + r) * row_bytes;
  }
  const int koff = g * M::kLaneBytes;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int64_t full = row_bytes - row_bytes % kSmallBatchBytes;   // whole batches
  int64_t k = 0;
  for (; k < full; k += kSmallBatchBytes) {
    typename M::frag a[U], w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w0[u] = M::load(bp0 + k + u * M::kStepBytes + koff);
      if constexpr (GATE_UP) w1[u] = M::load(bp1 + k + u * M::kStepBytes + koff);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = ap ? M::load(ap + k + u * M::kStepBytes + koff) : M::zero();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc0 = M::mma(a[u], w0[u], acc0);
      if constexpr (GATE_UP) acc1 = M::mma(a[u], w1[u], acc1);
    }
  }
  for (; k < row_bytes; k += M::kStepBytes) {   // tail steps (FP8 rows of 256 * odd bytes)
    const typename M::frag w0 = M::load(bp0 + k + koff);
    typename M::frag w1 = M::zero();
    if constexpr (GATE_UP) w1 = M::load(bp1 + k + koff);
    const typename M::frag a = ap ? M::load(ap + k + koff) : M::zero();
    acc0 = M::mma(a, w0, acc0);
    if constexpr (GATE_UP) acc1 = M::mma(a, w1, acc1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    if (row >= rows) continue;
    const int col = c0 + r;
    if constexpr (GATE_UP) {
      float gv = acc0[i], uv = acc1[i];
      if constexpr (FP8) {
        const float sx = a_scale[at.sorted_slot[row0 + row] / topk];
        gv = gv * sx * w_scale[(int64_t)e * 2 * Nout + col];
        uv = uv * sx * w_scale[(int64_t)e * 2 * Nout + Nout + col];
      }
      const float h = silu_f32(bf16_round(gv)) * bf16_round(uv);
      reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + col] =
          (uint16_t)f32_to_bf16_bits(h);
    } else {
      const int slot = at.sorted_slot[row0 + row];
      float y = acc0[i];
      if constexpr (FP8) y = y * a_scale[row0 + row] * w_scale[(int64_t)e * Nout + col];
      reinterpret_cast<float*>(out)[(int64_t)slot * Nout + col] = at.sorted_w[row0 + row] * y;
    }
  }
}

// K-split variant: a WG covers 16 h columns (gate/up: each lane streams a gate row and the
// matching up row) or 32 output columns (down: two 16-column groups, so a down workgroup streams as
// many weight bytes as a gate/up one; measured 0.516 -> 0.503 ms at T=32), and its waves (4 or 8,
// KSW) split K (many more workgroups than the column-tiled kernel, which matters when a handful
// of tokens touch few experts): wave w takes batches w, w + KSW, w + 2 KSW, ... of every row, so
// at any moment a workgroup reads one contiguous stretch of each row (0.5-1.5% faster than
// contiguous per-wave parts). Each wave keeps two batches of loads in flight (the next batch is
// issued before the current one's MFMAs); the partial tiles are summed in LDS in wave order
// (deterministic) and wave 0 runs the epilogue. Requires the rows to split into KSW x whole
// batches.
template <bool FP8>
struct KsBatch {
  static constexpr int kBytes = 256;   // bf16: 4 steps of 64 B; FP8: 2 steps of 128 B
};
template <>
struct KsBatch<true> {
  static constexpr int kBytes = 128;   // one 128-deep FP8 step (the quarter of 2560 is 640 B)
};

// KSW = waves splitting K: 8 for bf16 gate/up where its rows split into whole batches
// (shorter-lived workgroups, so less of the grid's tail runs part-empty: 0.996 -> 0.986 ms at
// T=32), else 4 (FP8 gate/up measured 6% slower with 8: its eighths of a row are 5 one-step
// batches).
template <bool GATE_UP, bool FP8, int KSW>
__global__ __launch_bounds__(64 * KSW) void grouped_small_ks_kernel(
    const unsigned char* __restrict__ A, const unsigned char* __restrict__ W,
    void* __restrict__ out, AlignTables at, int Kd, int Nout,
    int topk, const float* __restrict__ a_scale, const float* __restrict__ w_scale) {
  using M = SmallMath<FP8>;
  constexpr int U = KsBatch<FP8>::kBytes / M::kStepBytes;   // MFMA steps per batch
  constexpr int NACC = 2;   // gate/up: a gate and an up row per lane; down: two 16-column groups
  constexpr int kKsWaves = KSW;
  __shared__ floatx4 red[kKsWaves][NACC][64];
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * (GATE_UP ? 16 : 32);
  const int64_t row_bytes = (int64_t)Kd * M::kElemBytes;
  constexpr int64_t BB = KsBatch<FP8>::kBytes;
  const int64_t kq = row_bytes / kKsWaves, kbeg = wave * BB;   // batches wave, wave + KSW, ...

  const unsigned char* ap = nullptr;
  if (r < rows) {
    if constexpr (GATE_UP)
      ap = A + (int64_t)(at.sorted_slot[row0 + r] / topk) * row_bytes + kbeg;
    else
      ap = A + (int64_t)(row0 + r) * row_bytes + kbeg;
  }
  const unsigned char* bp0;
  const unsigned char* bp1 = nullptr;
  if constexpr (GATE_UP) {
    bp0 = W + ((int64_t)e * 2 * Nout + c0 + r) * row_bytes + kbeg;
    bp1 = W + ((int64_t)e * 2 * Nout + Nout + c0 + r) * row_bytes + kbeg;
  } else {
    bp0 = W + ((int64_t)e * Nout + c0 + r) * row_bytes + kbeg;
    bp1 = bp0 + 16 * row_bytes;
  }
  const int koff = g * M::kLaneBytes;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  typename M::frag a[2][U], w0[2][U], w1[2][U];
  auto load = [&](int buf, int64_t k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w0[buf][u] = M::load(bp0 + k + u * M::kStepBytes + koff);
      w1[buf][u] = M::load(bp1 + k + u * M::kStepBytes + koff);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      a[buf][u] = ap ? M::load(ap + k + u * M::kStepBytes + koff) : M::zero();
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc0 = M::mma(a[buf][u], w0[buf][u], acc0);
      acc1 = M::mma(a[buf][u], w1[buf][u], acc1);
    }
  };
  const int nb = (int)(kq / BB);
  constexpr int64_t SB = BB * KSW;   // bytes between a wave's batches
  load(0, 0);
  int i = 0;
  for (; i + 2 <= nb; i += 2) {   // two batches per trip so the buffers stay in registers
    load(1, (int64_t)(i + 1) * SB);
    mma(0);
    if (i + 2 < nb) load(0, (int64_t)(i + 2) * SB);
    mma(1);
  }
  if (i < nb) mma(0);   // odd count: batch nb-1 was loaded into buffer 0

  red[wave][0][lane] = acc0;
  red[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  floatx4 s0 = red[0][0][lane], s1 = red[0][1][lane];
#pragma unroll
  for (int w = 1; w < kKsWaves; ++w) {
    s0 += red[w][0][lane];
    s1 += red[w][1][lane];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * g + q;
    if (row >= rows) continue;
    const int col = c0 + r;
    if constexpr (GATE_UP) {
      float gv = s0[q], uv = s1[q];
      if constexpr (FP8) {
        const float sx = a_scale[at.sorted_slot[row0 + row] / topk];
        gv = gv * sx * w_scale[(int64_t)e * 2 * Nout + col];
        uv = uv * sx * w_scale[(int64_t)e * 2 * Nout + Nout + col];
      }
      const float h = silu_f32(bf16_round(gv)) * bf16_round(uv);
      reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + col] =
          (uint16_t)f32_to_bf16_bits(h);
    } else {
      const int slot = at.sorted_slot[row0 + row];
      const float wgt = at.sorted_w[row0 + row];
      float y0 = s0[q], y1 = s1[q];
      if constexpr (FP8) {
        const float sr = a_scale[row0 + row];
        y0 = y0 * sr * w_scale[(int64_t)e * Nout + col];
        y1 = y1 * sr * w_scale[(int64_t)e * Nout + col + 16];
      }
      float* const yrow = reinterpret_cast<float*>(out) + (int64_t)slot * Nout;
      yrow[col] = wgt * y0;
      yrow[col + 16] = wgt * y1;
    }
  }
}

}  // namespace beam
