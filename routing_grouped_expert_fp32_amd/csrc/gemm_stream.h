// Grouped bf16 GEMM for large row blocks (gfx950): weights streamed into registers, token rows in
// an LDS ring.
//
// Near the HBM/MFMA ridge (about 256 rows per expert) the kernel must stream every weight byte once
// at close to HBM rate while the MFMAs keep up. Design:
//   * WG tile: up to 256 rows of one expert x 256 weight columns (gate/up: 128 gate columns and the
//     128 matching up columns). Wave w owns 64 of the columns (gate/up: 32 gate + the 32 matching up
//     columns) for all rows: 16 x 4 MFMA tiles of 16x16 (v_mfma_f32_16x16x32_bf16), 256 fp32
//     accumulators per lane. Waves share no weight bytes.
//   * Weights: each lane loads its MFMA operand fragments (16 bytes of one weight row) straight from
//     HBM into a register ring kBP 32-deep K steps ahead, so every wave keeps 4 * kBP KB in flight.
//   * Token rows: one 256-row x 64-deep stage (32 KB) per 2 K steps, brought by global_load_lds into
//     a kAStages ring (XOR-swizzled 128-byte rows, as in the pipelined kernel) and read as
//     fragments by all four waves.
//   * Row sub-tiles past the block's rows skip their MFMAs; all waves skip the same ones (they share
//     the rows), in steps of 4 sub-tiles (64 rows).
//   * XCD-aware tile order as in the pipelined kernel.
#pragma once
#include <type_traits>

#include "common.h"
#include "gemm_pipe.h"

namespace beam {

constexpr int kSBM = 256;
constexpr int kSBP = 8;                      // weight-register ring depth in 32-deep K steps
constexpr int kSAStages = 4;                 // token-row LDS stages (64 deep each)
constexpr int kSAStageBytes = kSBM * 128;    // 32 KB
constexpr int kSALoadsPerWave = kSBM / 8 / 4;   // 1 KB direct loads per wave per stage (8)
static_assert(kSBP % 2 == 0, "ring slots must align with 64-deep token stages");

// s_waitcnt vmcnt(n) for a runtime n (multiple of 4, at most 60)
__device__ __forceinline__ void wait_vmcnt4(int n) {
  switch (n >> 2) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(16)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(20)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(24)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(28)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(32)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(36)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(40)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(44)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(48)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vmcnt_imm(52)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vmcnt_imm(56)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(60)); break;
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void grouped_stream_kernel(
    const unsigned char* __restrict__ A, const unsigned char* __restrict__ W,
    const float* __restrict__ topk_w, void* __restrict__ out, AlignTables at, int Kd, int Nout,
    int topk, int n_ctiles) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSAStages * kSAStageBytes];
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
  const int r = lane & 15, g = lane >> 4;
  const int64_t row_bytes = (int64_t)Kd * 2;
  const int ns = Kd / 32;                     // 32-deep K steps
  const int nst = ns / 2;                     // 64-deep token stages

  // ---- token-row direct loads: wave w covers block rows [64w, 64w+64) in 8 loads of 8 rows
  const int lrow = lane >> 3;
  const int gchunk = (lane & 7) ^ lrow;
  const unsigned char* asrc[kSALoadsPerWave];
#pragma unroll
  for (int q = 0; q < kSALoadsPerWave; ++q) {
    int rr = (wave * kSALoadsPerWave + q) * 8 + lrow;
    if (rr >= rows) rr = rows - 1;             // padding rows re-read a valid row (discarded)
    const int64_t arow =
        GATE_UP ? (int64_t)(at.sorted_slot[row0 + rr] / topk) : (int64_t)(row0 + rr);
    asrc[q] = A + arow * row_bytes + gchunk * 16;
  }
  auto issue_a = [&](int stage) {
    unsigned char* base = smem + (stage % kSAStages) * kSAStageBytes;
    const int kb = stage * 128;
#pragma unroll
    for (int q = 0; q < kSALoadsPerWave; ++q)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(asrc[q] + kb),
                                       (lds_void_t*)(base + (wave * kSALoadsPerWave + q) * 1024),
                                       16, 0, 0);
  };

  // ---- weight rows of this lane for its 4 N sub-tiles: gate/up n = 0,1 gate, n = 2,3 up
  const unsigned char* wsrc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    int64_t wrow;
    if constexpr (GATE_UP)
      wrow = (int64_t)e * 2 * Nout + (n < 2 ? 0 : Nout) + 128 * j + 32 * wave + 16 * (n & 1) + r;
    else
      wrow = (int64_t)e * Nout + 256 * j + 64 * wave + 16 * n + r;
    wsrc[n] = W + wrow * row_bytes + g * 16;
  }
  bf16x8 bring[kSBP][4];

  floatx4 acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: token stages 0..kSAStages-2, weight steps 0..kSBP-1
#pragma unroll
  for (int s = 0; s < kSAStages - 1; ++s)
    if (s < nst) issue_a(s);
#pragma unroll
  for (int u = 0; u < kSBP; ++u)
#pragma unroll
    for (int n = 0; n < 4; ++n)
      bring[u][n] = (u < ns) ? *reinterpret_cast<const bf16x8*>(wsrc[n] + u * 64) : bf16x8{};

  // VMEM ops a wave issues at step s (in order): token loads for stage s/2 + kSAStages - 1 when s
  // is even (kSALoadsPerWave), then weight loads for step s + kSBP (4).
  auto ops_at = [&](int s) {
    int n = 0;
    if ((s & 1) == 0 && s / 2 + kSAStages - 1 < nst) n += kSALoadsPerWave;
    if (s + kSBP < ns) n += 4;
    return n;
  };
  const int frag_off0 = r * 128 + (((0 + g) ^ (r & 7)) << 4);
  const int frag_off1 = r * 128 + (((4 + g) ^ (r & 7)) << 4);

  auto kloop = [&](auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;   // valid 16-row sub-tiles (multiple of 4)
    for (int s0 = 0; s0 < ns; s0 += kSBP) {
#pragma unroll
      for (int u = 0; u < kSBP; ++u) {
        const int s = s0 + u;
        if (s >= ns) break;
        if ((u & 1) == 0) {
          // token stage s/2 must be complete: ops issued after its loads may stay in flight.
          // Its loads were issued at step s0' = s - 2*(kSAStages-1) (or in the prologue).
          const int kt = s >> 1;
          int after = 0;
          if (kt >= kSAStages - 1) {
            const int si = 2 * (kt - (kSAStages - 1));   // step that issued this stage
            after = (si + kSBP < ns) ? 4 : 0;             // that step's weight loads
            for (int q = si + 1; q < s; ++q) after += ops_at(q);
          } else {
            // issued in the prologue: younger prologue token stages, all prologue weight steps,
            // and everything issued by steps 0 .. s-1
            for (int q = kt + 1; q < kSAStages - 1 && q < nst; ++q) after += kSALoadsPerWave;
            after += 4 * min(kSBP, ns);
            for (int q = 0; q < s; ++q) after += ops_at(q);
          }
          wait_vmcnt4(min(after, 60));
          lds_ring_barrier();
          if (kt + kSAStages - 1 < nst) issue_a(kt + kSAStages - 1);
        }
        const unsigned char* sa = smem + ((s >> 1) % kSAStages) * kSAStageBytes;
        const int fo = (u & 1) ? frag_off1 : frag_off0;
        bf16x8 af[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) af[i] = *reinterpret_cast<const bf16x8*>(sa + i * 2048 + fo);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bring[u][n], acc[i][n], 0,
                                                                0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (s + kSBP < ns) {
#pragma unroll
          for (int n = 0; n < 4; ++n)
            bring[u][n] = *reinterpret_cast<const bf16x8*>(wsrc[n] + (s + kSBP) * 64);
        }
      }
    }
  };
  const int nsub = (rows + 15) >> 4;
  if (nsub > 12)
    kloop(std::integral_constant<int, 16>{});
  else if (nsub > 8)
    kloop(std::integral_constant<int, 12>{});
  else if (nsub > 4)
    kloop(std::integral_constant<int, 8>{});
  else
    kloop(std::integral_constant<int, 4>{});

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = i * 16 + 4 * g + q;
      if (row >= rows) continue;
      if constexpr (GATE_UP) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float h = silu_f32(bf16_round(acc[i][n][q])) * bf16_round(acc[i][n + 2][q]);
          const int hcol = 128 * j + 32 * wave + 16 * n + r;
          reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + hcol] =
              (uint16_t)f32_to_bf16_bits(h);
        }
      } else {
        const int slot = at.sorted_slot[row0 + row];
        const float wgt = topk_w[slot];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int col = 256 * j + 64 * wave + 16 * n + r;
          reinterpret_cast<float*>(out)[(int64_t)slot * Nout + col] = wgt * acc[i][n][q];
        }
      }
    }
  }
}

}  // namespace beam
