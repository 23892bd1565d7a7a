// Pipelined grouped bf16 GEMM for large row blocks (gfx950): direct-to-LDS loads.
//
// Used by the gate/up (fused SwiGLU epilogue) and down (weighted epilogue) steps when experts carry
// many rows (prefill-sized batches). Design:
//   * WG tile: up to 256 rows of one expert x 256 weight columns (gate/up: 128 gate columns and the
//     128 matching up columns); 4 waves in a 2 x 2 grid, wave tile 128 x 128 (8 x 8 MFMA
//     16x16x32 tiles, 256 fp32 accumulators per lane).
//   * K is staged kPBK deep. Global -> LDS with global_load_lds_dwordx4: one wave instruction lands
//     1 KB contiguously in LDS = kPRowsPerLoad rows x kPBK*2 bytes (8 rows x 128 B at kPBK = 64, so
//     every instruction reads whole 128-byte lines); each lane fetches the 16-byte chunk that
//     belongs at its LDS slot. Chunk c of row r is stored at chunk position c ^ swz(r), so the 16
//     rows a fragment read touches fall on distinct banks.
//   * kPStages LDS stages; loads for stage kt+kPStages-1 are issued right after the barrier of
//     stage kt; each wave waits (s_waitcnt vmcnt) only for its own loads of the stage it reads.
//   * Row sub-tiles are dealt to the two wave rows alternately (wave row wm takes 16-row sub-tiles
//     wm, wm+2, ...); a wave runs one of four K-loop bodies (2, 4, 6 or 8 sub-tiles), chosen by how
//     many of its sub-tiles hold rows, so a partly filled block costs about its rows.
//   * Tile order is XCD-aware: workgroup L runs on XCD L % 8; the (block, column-tile) space is cut
//     into 8 contiguous ranges, one per XCD, walked column-tile fastest, so the workgroups sharing
//     a block's token rows — and the blocks of one expert sharing weight tiles — run together on
//     one XCD's L2.
#pragma once
#include <type_traits>

#include "common.h"

namespace beam {

constexpr int kPBM = 256;                       // max rows per block
constexpr int kPBN = 256;                       // weight columns per WG tile
constexpr int kPBK = 64;                        // K per stage
constexpr int kPStages = 2;
constexpr int kPRowBytes = kPBK * 2;            // bytes of one row in one stage
constexpr int kPChunks = kPBK / 8;              // 16-byte chunks per row per stage
constexpr int kPRowsPerLoad = 64 / kPChunks;    // rows covered by one 1 KB wave load
constexpr int kPLoadsA = kPBM / kPRowsPerLoad;  // wave loads per stage for the token rows
constexpr int kPLoadsB = kPBN / kPRowsPerLoad;  // ... and for the weight rows
constexpr int kPLoadsPerWave = (kPLoadsA + kPLoadsB) / 4;
constexpr int kPStageBytes = (kPBM + kPBN) * kPRowBytes;
static_assert(kPBK == 32 || kPBK == 64, "swizzle below is defined for 64- and 128-byte rows");
static_assert(kPStages >= 2 && kPStageBytes * kPStages <= 160 * 1024, "LDS budget");
static_assert(kPLoadsPerWave * 3 < 64, "vmcnt range");

// chunk-position swizzle: 8 consecutive rows land their chunk c on 8 distinct 16-byte positions
__device__ __forceinline__ int pswz(int r) { return kPChunks == 8 ? (r & 7) : ((r >> 1) & 3); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate (gfx9 encoding) waiting until at most n vector-memory ops are outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without the memory fence __syncthreads() adds (that fence waits for every
// outstanding load, which would drain the prefetch). The empty asm statements keep the compiler
// from moving memory accesses across it; LDS written by direct loads is visible once the issuing
// wave's vmcnt wait has passed and every wave has reached the barrier.
__device__ __forceinline__ void lds_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void grouped_pipe_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ W,
                                                              const float* __restrict__ topk_w,
                                                              void* __restrict__ out,
                                                              AlignTables at, int Kd, int Nout,
                                                              int topk, int n_ctiles) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPStages * kPStageBytes];
  // ---- tile assignment (XCD-aware) ----
  const int L = blockIdx.x;
  const int xcd = L & 7, local = L >> 3;
  const int total = at.n_blocks[0] * n_ctiles;
  const int per = (total + 7) >> 3;
  if (local >= per) return;
  const int v = xcd * per + local;
  if (v >= total) return;
  const int b = v / n_ctiles, j = v % n_ctiles;
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- direct-load sources. Wave w issues token-row loads a = w*LA .. and weight-row loads
  // q = w*LB ..; load a covers block rows [a*RPL, (a+1)*RPL): lane -> row a*RPL + lane/CH, chunk
  // slot lane%CH, global chunk = slot ^ swz(row).
  constexpr int LA = kPLoadsA / 4, LB = kPLoadsB / 4;
  const int lrow = lane / kPChunks;
  const int gchunk = (lane % kPChunks) ^ pswz(lrow);
  const uint16_t* asrc[LA];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    int rr = (wave * LA + q) * kPRowsPerLoad + lrow;   // block row 0..255
    if (rr >= rows) rr = rows - 1;                      // padding rows re-read a valid row
    const int64_t arow =
        GATE_UP ? (int64_t)(at.sorted_slot[row0 + rr] / topk) : (int64_t)(row0 + rr);
    asrc[q] = A + arow * Kd + gchunk * 8;
  }
  // weight tile row br = (wave*LB + q)*RPL + lrow; gate/up tiles: rows [0,128) gate, [128,256) up.
  // A wave's LB loads cover 64 consecutive tile rows, all in one half.
  const int br0 = wave * LB * kPRowsPerLoad + lrow;
  int64_t wrow0;
  if constexpr (GATE_UP)
    wrow0 = (int64_t)e * 2 * Nout + (br0 < 128 ? 128 * j + br0 : Nout + 128 * j + (br0 - 128));
  else
    wrow0 = (int64_t)e * Nout + 256 * j + br0;
  const uint16_t* bsrc = W + wrow0 * Kd + gchunk * 8;
  const int64_t bstep = (int64_t)kPRowsPerLoad * Kd;   // elements between consecutive loads

  auto issue = [&](int stage_k, int buf) {
    unsigned char* base = smem + buf * kPStageBytes;
#pragma unroll
    for (int q = 0; q < LA; ++q)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(asrc[q] + stage_k),
                                       (lds_void_t*)(base + (wave * LA + q) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < LB; ++q)
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(bsrc + q * bstep + stage_k),
          (lds_void_t*)(base + kPBM * kPRowBytes + (wave * LB + q) * 1024), 16, 0, 0);
  };

  floatx4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[i][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kd / kPBK;
#pragma unroll
  for (int s = 0; s < kPStages - 1; ++s)
    if (s < nk) issue(s * kPBK, s);

  // fragment byte offset of this lane inside a 16-row group for 32-deep step h of a stage:
  // row r = lane % 16, chunk 4h + lane/16 (swizzled)
  const int r = lane & 15, g = lane >> 4;
  int frag_off[kPBK / 32];
#pragma unroll
  for (int h = 0; h < kPBK / 32; ++h) frag_off[h] = r * kPRowBytes + (((4 * h + g) ^ pswz(r)) << 4);

  auto kloop = [&](auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;
    for (int kt = 0; kt < nk; ++kt) {
      const int younger = min(kPStages - 2, nk - 1 - kt);   // stages issued after this one
      switch (younger) {
        case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPLoadsPerWave)); break;
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPLoadsPerWave)); break;
      }
      lds_ring_barrier();
      if (kt + kPStages - 1 < nk)
        issue((kt + kPStages - 1) * kPBK, (kt + kPStages - 1) % kPStages);
      const unsigned char* sa = smem + (kt % kPStages) * kPStageBytes;
      const unsigned char* sb = sa + kPBM * kPRowBytes;
#pragma unroll
      for (int h = 0; h < kPBK / 32; ++h) {
        bf16x8 bw[8], af[NV];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          int grp;   // 16-row group of the weight tile feeding N sub-tile n of this wave
          if constexpr (GATE_UP)
            grp = n < 4 ? 4 * wn + n : 8 + 4 * wn + (n - 4);
          else
            grp = 8 * wn + n;
          bw[n] = *reinterpret_cast<const bf16x8*>(sb + grp * 16 * kPRowBytes + frag_off[h]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)   // 16-row sub-tile wm + 2i of the block
          af[i] = *reinterpret_cast<const bf16x8*>(sa + (wm + 2 * i) * 16 * kPRowBytes +
                                                   frag_off[h]);
        __builtin_amdgcn_sched_barrier(0);   // all reads ahead of the MFMA chain
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int n = 0; n < 8; ++n)
            acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[n], acc[i][n], 0, 0, 0);
      }
    }
  };
  // valid sub-tiles of this wave: mt = wm + 2i < ceil(rows / 16); bodies for 2, 4, 6, 8
  const int nsub = (rows + 15) >> 4;
  const int nv = nsub > wm ? min(8, (nsub - wm + 1) >> 1) : 0;
  if (nv > 6)
    kloop(std::integral_constant<int, 8>{});
  else if (nv > 4)
    kloop(std::integral_constant<int, 6>{});
  else if (nv > 2)
    kloop(std::integral_constant<int, 4>{});
  else
    kloop(std::integral_constant<int, 2>{});

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int mt = wm + 2 * i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = mt * 16 + 4 * g + q;
      if (row >= rows) continue;
      if constexpr (GATE_UP) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const float h = silu_f32(bf16_round(acc[i][n][q])) * bf16_round(acc[i][n + 4][q]);
          const int hcol = 128 * j + 64 * wn + 16 * n + r;
          reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + hcol] =
              (uint16_t)f32_to_bf16_bits(h);
        }
      } else {
        const int slot = at.sorted_slot[row0 + row];
        const float wgt = topk_w[slot];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int col = 256 * j + 128 * wn + 16 * n + r;
          reinterpret_cast<float*>(out)[(int64_t)slot * Nout + col] = wgt * acc[i][n][q];
        }
      }
    }
  }
}

}  // namespace beam
