// Weight-streaming grouped GEMM for small row blocks (<= 16 rows; decode-sized batches), gfx950.
//
// At decode each touched expert carries a handful of rows, so every weight byte is used once or
// twice: the kernels are HBM streams. The K-split kernel (below) is the one decode shapes use;
// the column-tiled kernel covers rows that do not split into whole batches: WG = 4 waves x 16
// output columns, each lane streaming its weight row(s) straight from HBM into MFMA operand
// registers, 512 bytes of every row per batch with all of a batch's loads issued before its MFMAs
// (a row's last bytes short of a batch go one MFMA step at a time). Token rows past the block's
// rows are zero operands (the K-split kernel re-reads row 0 instead); their results are
// discarded.
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
// contiguous per-wave parts). Weight batches travel HBM -> LDS through non-temporal direct loads
// of whole 128-byte lines (6.3 -> 6.9 TB/s on the decode gate/up stream against register loads,
// which can fetch only half a line per row per instruction in MFMA operand order); each wave
// owns two LDS slots and keeps the next batch in flight while it computes the current one, and
// reads back only what it loaded itself, so no workgroup barrier is needed. The partial tiles
// are summed in LDS in wave order (deterministic) and wave 0 runs the epilogue. Requires the
// rows to split into KSW x whole batches.
template <bool FP8>
struct KsBatch {
  static constexpr int kBytes = 256;   // bf16: 4 steps of 64 B
};
template <>
struct KsBatch<true> {
  static constexpr int kBytes = 128;   // one 128-deep FP8 step (the quarter of 2560 is 640 B)
};

// KSW = waves splitting K, 4 for every launch: with the LDS slots, 8-wave bf16 gate/up workgroups
// (144 KB of LDS, one per CU) measured 0.897 ms at T=32 against 0.875 ms for two 4-wave ones per
// CU (whose starts and ends overlap); FP8 gate/up was 6% slower with 8 already with register loads.
template <bool GATE_UP, bool FP8, int KSW>
__global__ __launch_bounds__(64 * KSW) void grouped_small_ks_kernel(
    const unsigned char* __restrict__ A, const unsigned char* __restrict__ W,
    void* __restrict__ out, AlignTables at, int Kd, int Nout,
    int topk, const float* __restrict__ a_scale, const float* __restrict__ w_scale) {
  using M = SmallMath<FP8>;
  constexpr int BB = KsBatch<FP8>::kBytes;
  constexpr int U = BB / M::kStepBytes;   // MFMA steps per batch
  constexpr int LINES = BB / 128;         // 128-byte lines of each weight row per batch
  constexpr int NLD = 4 * LINES;          // direct loads per batch: 32 rows, 8 rows per load
  constexpr int A_OPS = U * (M::kLaneBytes / 16);   // token-row loads per batch
  constexpr int kSlot = NLD * 1024;
  constexpr int kRing = KSW * 2 * kSlot;  // two batch slots per wave
  // one LDS array: the weight rings, then the K-split partial tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRing + KSW * 2 * 64 * 16];
  floatx4(*red)[2][64] = reinterpret_cast<floatx4(*)[2][64]>(smem + kRing);
  const int b = blockIdx.y;
  if (b >= at.n_blocks[0]) return;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * (GATE_UP ? 16 : 32);
  const int64_t row_bytes = (int64_t)Kd * M::kElemBytes;
  const int nb = (int)(row_bytes / KSW / BB);   // batches of this wave: wave, wave + KSW, ...
  constexpr uint32_t SB = (uint32_t)BB * KSW;   // bytes between a wave's batches
  const uint32_t kbeg = (uint32_t)wave * BB;

  // token rows into registers through a buffer (x, under 4 GiB, or the block's rows of h);
  // padding rows re-read row 0 (their results are discarded)
  const int rr = r < rows ? r : 0;
  const unsigned char* abase = GATE_UP ? A : A + (int64_t)row0 * row_bytes;
  const uint32_t abytes = GATE_UP ? 0xffffffffu : (uint32_t)(rows * row_bytes);
  const uint32_t aoff =
      (uint32_t)((GATE_UP ? (int64_t)(at.sorted_slot[row0 + rr] / topk) : (int64_t)rr) *
                 row_bytes) + kbeg + g * M::kLaneBytes;

  // weight rows of the workgroup, 0..31: gate/up 16 gate rows then the 16 matching up rows; down
  // 32 output columns. They arrive through non-temporal direct loads of whole 128-byte lines (a
  // line fetched by halves into registers is fetched twice once it bypasses L2 retention):
  // load (group rg of 8 rows, line ln) lands 1 KB in LDS, lane -> row 8 rg + lane / 8, LDS chunk
  // lane % 8 holding line chunk (lane % 8) ^ (row % 8), so a fragment read of 16 rows is
  // conflict-free. Buffers: the expert's gate half and up half (down: its matrix).
  const unsigned char* wb0 = W + (int64_t)e * (GATE_UP ? 2 : 1) * Nout * row_bytes;
  const unsigned char* wb1 = GATE_UP ? wb0 + (int64_t)Nout * row_bytes : wb0;
  const uint32_t wbytes = (uint32_t)(Nout * row_bytes);
  const int lrow = lane >> 3, gch = (lane & 7) ^ lrow;
  uint32_t voff[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    const int wr = 8 * rg + lrow;
    voff[rg] = (uint32_t)((c0 + (GATE_UP ? (wr & 15) : wr)) * row_bytes) + kbeg + gch * 16;
  }
  unsigned char* const ring = smem + wave * 2 * kSlot;
  // LDS byte offset of this lane's 16-byte piece `piece` (0..7 within a line) of weight row wr
  auto frag_at = [&](int wr, int ln, int piece) {
    return ((wr >> 3) * LINES + ln) * 1024 + (wr & 7) * 128 + ((piece ^ (wr & 7)) << 4);
  };

  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  typename M::frag a[2][U];
  // batch i of this wave into slot buf. live == false issues the same loads against empty
  // buffers (no memory access, zeros): every trip then issues the same number of loads, so the
  // wait counts below are exact on every path.
  auto issue = [&](int buf, int i, bool live) {
    const uint32_t kb = (uint32_t)i * SB;
    const uint32_t ab = __builtin_amdgcn_readfirstlane(live ? abytes : 0u);
    const uint32_t wbb = __builtin_amdgcn_readfirstlane(live ? wbytes : 0u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (FP8) {
        const u32x4 lo = buffer_load16<0>(abase, ab, aoff, kb + u * M::kStepBytes);
        const u32x4 hi = buffer_load16<0>(abase, ab, aoff + 16, kb + u * M::kStepBytes);
        a[buf][u] = typename M::frag{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        a[buf][u] = __builtin_bit_cast(bf16x8, buffer_load16<0>(abase, ab, aoff,
                                                                kb + u * M::kStepBytes));
      }
    }
    unsigned char* slot = ring + buf * kSlot;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int ln = 0; ln < LINES; ++ln)
        buffer_load_lds16<kCachePolicyNT>(rg < 2 ? wb0 : wb1, wbb, voff[rg] + ln * 128, kb,
                                          (lds_void_t*)(slot + (rg * LINES + ln) * 1024));
  };
  auto compute = [&](int buf) {
    const unsigned char* slot = ring + buf * kSlot;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ln = (u * M::kStepBytes) / 128, p0 = (u * M::kStepBytes) % 128 / 16;
      typename M::frag w0, w1;
      if constexpr (FP8) {
        const intx4 l0 = *reinterpret_cast<const intx4*>(slot + frag_at(r, ln, p0 + 2 * g));
        const intx4 h0 = *reinterpret_cast<const intx4*>(slot + frag_at(r, ln, p0 + 2 * g + 1));
        const intx4 l1 = *reinterpret_cast<const intx4*>(slot + frag_at(16 + r, ln, p0 + 2 * g));
        const intx4 h1 =
            *reinterpret_cast<const intx4*>(slot + frag_at(16 + r, ln, p0 + 2 * g + 1));
        w0 = typename M::frag{l0.x, l0.y, l0.z, l0.w, h0.x, h0.y, h0.z, h0.w};
        w1 = typename M::frag{l1.x, l1.y, l1.z, l1.w, h1.x, h1.y, h1.z, h1.w};
      } else {
        w0 = *reinterpret_cast<const bf16x8*>(slot + frag_at(r, ln, p0 + g));
        w1 = *reinterpret_cast<const bf16x8*>(slot + frag_at(16 + r, ln, p0 + g));
      }
      acc0 = M::mma(a[buf][u], w0, acc0);
      acc1 = M::mma(a[buf][u], w1, acc1);
    }
  };
  // Each wave reads only what it loaded itself: no barrier, its own vmcnt wait makes a slot
  // visible; a slot is refilled only after the reads of its previous batch have returned.
  constexpr int kBatchOps = A_OPS + NLD;
  issue(0, 0, true);
  int i = 0;
  for (; i + 2 <= nb; i += 2) {   // two batches per trip so the token fragments stay in registers
    issue(1, i + 1, true);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBatchOps));   // batch i has landed
    compute(0);
    __builtin_amdgcn_s_waitcnt(kLgkmZero);   // slot 0's reads are done before it is refilled
    __builtin_amdgcn_sched_barrier(0);
    issue(0, i + 2, i + 2 < nb);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBatchOps));   // batch i + 1 has landed
    compute(1);
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i < nb) {   // odd count: batch nb-1 was issued into slot 0
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compute(0);
  }

  red[wave][0][lane] = acc0;
  red[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  floatx4 s0 = red[0][0][lane], s1 = red[0][1][lane];
#pragma unroll
  for (int w = 1; w < KSW; ++w) {
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
