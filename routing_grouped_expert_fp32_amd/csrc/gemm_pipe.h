// Pipelined grouped GEMM for large row blocks (gfx950): direct-to-LDS loads, bf16 or FP8 E4M3.
//
// Used by the gate/up (fused SwiGLU epilogue) and down (weighted epilogue) steps when experts carry
// many rows (prefill-sized batches). Design:
//   * WG tile: 320 rows of one expert x 256 weight columns (gate/up: 128 gate columns and the 128
//     matching up columns), 8 waves in a 4 x 2 grid, two per SIMD, so one wave's barrier and LDS
//     waits overlap the other's MFMAs. Wave tile 80 x 128 (160 fp32 accumulators per lane). bf16
//     uses v_mfma_f32_16x16x32_bf16; FP8 the 16x16x128 f8f6f4 MFMA with unit block scales
//     (operands OCP E4M3FN), its 8-register weight fragments read in two halves.
//   * Each stage carries 128 bytes of every row (64 bf16 or 128 FP8 values). Global -> LDS with
//     buffer_load_dwordx4 ... lds: one wave instruction lands 1 KB = 8 rows x 128 B (whole cache
//     lines) contiguously in LDS; each lane fetches the 16-byte chunk that belongs at its LDS slot.
//     Chunk c of row r is stored at chunk position c ^ (r & 7), so the 16 rows a fragment read
//     touches fall on distinct banks. Weight loads go through a buffer covering the expert's gate
//     or up half (down: the expert's matrix), the down step's token loads through one covering
//     the block's rows (out-of-range lanes would read zero, never fault).
//   * Separate LDS rings: token rows (L2-resident, short latency) 2 x 40 KB and weights (streamed
//     from HBM) 2 x 32 KB, both issued one stage ahead; each stage begins with a wait for the
//     wave's own loads and a workgroup barrier.
//   * Row sub-tiles are dealt to the wave rows in turn (wave row wm of 4 takes 16-row sub-tiles
//     wm, wm+4, ...); a wave runs one of four K-loop bodies, chosen by how many of its sub-tiles
//     hold rows, so a partly filled block costs about its rows.
//   * Tile order is XCD-aware: workgroup L runs on XCD L % 8; the (block, column-tile) space is cut
//     into 8 contiguous ranges, one per XCD, walked column-tile fastest, so the workgroups sharing
//     a block's token rows run together on one XCD's L2 (and consecutive blocks of one expert run
//     on the same XCD). An expert with several blocks (skewed batches, the dense layer) has them
//     walked in groups of four, column-tile major inside a group, so four blocks share each weight
//     stage in L2 as well.
// Epilogues: gate/up  h = bf16( silu(bf16(g)) * bf16(u) ), g/u dequantised first for FP8
//            (acc * token scale * output-channel scale); down  Y[slot] = topk_w[slot] * y (FP32),
//            y = acc (* row scale * output-channel scale for FP8). The epilogue operands (down: each
//            row's slot id and routing weight; FP8: the row or token scales and the tile's output-
//            channel scales) are loaded into LDS at the start, behind the first stage's loads, so
//            the epilogue issues stores only (12-16% of the down GEMM's time went to the
//            epilogue's dependent loads and stores).
#pragma once
#include <type_traits>

#include "device_common.h"

namespace beam {

constexpr int kPBN = 256;                       // weight columns per WG tile
constexpr int kPRowBytes = 128;                 // bytes of one row in one stage
constexpr int kPChunks = kPRowBytes / 16;       // 16-byte chunks per row per stage
constexpr int kPRowsPerLoad = 64 / kPChunks;    // rows covered by one 1 KB wave load
static_assert(kPChunks == 8, "swizzle below is defined for 128-byte rows");

// Block shape, both element types: 320 rows (every expert of a 256-rows-per-expert batch fits one
// block, so its weights stream once and the grid has one workgroup per expert and column tile),
// 8 waves (4 x 2, wave tile 80 x 128, 160 accumulators, two waves per SIMD), token rows 2 x 40 KB +
// weights 2 x 32 KB, both issued one stage ahead (144 KB of LDS).
template <bool FP8>
struct PipeCfg {
  static constexpr int BM = 320;
  static constexpr int WAVES = 8;
  static constexpr int AST = 2, BST = 2;
  static constexpr int kLoadsA = BM / kPRowsPerLoad;    // wave loads per stage, token rows
  static constexpr int kLoadsB = kPBN / kPRowsPerLoad;  // ... and weight rows
  static constexpr int kAStageBytes = BM * kPRowBytes;
  static constexpr int kBStageBytes = kPBN * kPRowBytes;
  static constexpr int kLdsBytes = AST * kAStageBytes + BST * kBStageBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kLoadsA % WAVES == 0 && kLoadsB % WAVES == 0, "loads split evenly over waves");
  static_assert((kLoadsA + kLoadsB) / WAVES < 64, "vmcnt range");
};

// blocks of one expert whose tiles are interleaved (tile order, below): with 32 CUs per XCD, 4
// blocks x 8 column tiles run at once, sharing each weight stage 4 ways and each token-row stage
// 8 ways in the XCD's L2
constexpr int kPGroup = 4;

// Workgroup barrier without the memory fence __syncthreads() adds (that fence waits for every
// outstanding load, which would drain the prefetch). The empty asm statements keep the compiler
// from moving memory accesses across it; LDS written by direct loads is visible once the issuing
// wave's vmcnt wait has passed and every wave has reached the barrier.
__device__ __forceinline__ void lds_ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool FP8>
struct PipeMath;
template <>
struct PipeMath<false> {   // bf16: two 32-deep steps per stage, one 16-byte read per fragment
  using frag = bf16x8;
  static constexpr int kSteps = 2, kReads = 1, kElemBytes = 2;
  __device__ static int chunk(int step, int g, int) { return 4 * step + g; }
  __device__ static frag read(const unsigned char* p, const int* off) {
    return *reinterpret_cast<const bf16x8*>(p + off[0]);
  }
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct PipeMath<true> {    // FP8: one 128-deep step per stage, two 16-byte reads per fragment
  using frag = intx8;
  static constexpr int kSteps = 1, kReads = 2, kElemBytes = 1;
  __device__ static int chunk(int, int g, int half) { return 2 * g + half; }
  __device__ static frag read(const unsigned char* p, const int* off) {
    const intx4 lo = *reinterpret_cast<const intx4*>(p + off[0]);
    const intx4 hi = *reinterpret_cast<const intx4*>(p + off[1]);
    return frag{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  __device__ static floatx4 mma(frag a, frag b, floatx4 c) {
    // formats 0/0 = E4M3 for both operands; E8M0 block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// A: token rows (gate/up: x, gathered through sorted_slot; down: h in sorted-row order).
// W: weights [E][rows][Kd]. Kd in elements. a_scale / w_scale: FP8 dequantisation scales
// (gate/up: per token / per weight row; down: per sorted row / per weight row), unused for bf16.
template <bool GATE_UP, bool FP8>
__global__ __launch_bounds__(64 * PipeCfg<FP8>::WAVES, 1) void grouped_pipe_kernel(
    const unsigned char* __restrict__ A, const unsigned char* __restrict__ W,
    void* __restrict__ out, AlignTables at, int Kd, int Nout,
    int topk, int n_ctiles, const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    int ksplit) {
  using M = PipeMath<FP8>;
  using C = PipeCfg<FP8>;
  constexpr int WAVES = C::WAVES;
  // one LDS array (a second __shared__ object makes the compiler wait for every direct load
  // right after issuing it): rings, then the epilogue's operands
  constexpr int kEpiBytes = GATE_UP ? (FP8 ? 12 * C::BM + 4 * kPBN : 0)
                                    : (FP8 ? 12 * C::BM + 4 * kPBN : 8 * C::BM);
  static_assert(C::kLdsBytes + kEpiBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kLdsBytes + kEpiBytes];
  unsigned char* const aring = smem;
  unsigned char* const bring = smem + C::AST * C::kAStageBytes;
  // ---- tile assignment (XCD-aware) ----
  const int L = blockIdx.x;
  const int xcd = L & 7, local = L >> 3;
  const int tiles = at.n_blocks[0] * n_ctiles;
  const int total = tiles * ksplit;
  const int per = (total + 7) >> 3;
  if (local >= per) return;
  const int v = xcd * per + local;
  if (v >= total) return;
  // K split (down only): part ksp of ksplit covers stages [ksp * nk, (ksp + 1) * nk) of the row
  // and writes its partial sums to output row slot * ksplit + ksp
  const int ksp = v / tiles, vt = v - ksp * tiles;
  // An expert's blocks form groups of up to kPGroup consecutive blocks; a group's tiles are walked
  // column-tile major, so the blocks that read one weight column tile run side by side on one
  // XCD and that tile streams from HBM about once per group instead of once per block. A
  // one-block group is walked as before (its column tiles in order, sharing the token rows).
  int b, j;
  bool shared_w;   // the tile's weight stages are read by other blocks of its group too
  {
    const int bn = vt / n_ctiles;                        // block in natural (column-fastest) order
    const int en = at.blk_expert[bn];
    const int e_rows0 = at.expert_off[en];
    const int ib = (at.blk_row0[bn] - e_rows0) / C::BM;  // block index within its expert
    const int nb = (at.expert_off[en + 1] - e_rows0 + C::BM - 1) / C::BM;
    const int g0 = ib - ib % kPGroup;
    const int sz = min(kPGroup, nb - g0);
    const int off = vt - (bn - (ib - g0)) * n_ctiles;   // tile within the group
    j = off / sz;
    b = bn - (ib - g0) + off % sz;
    shared_w = sz > 1;
  }
  const int e = at.blk_expert[b], row0 = at.blk_row0[b], rows = at.blk_rows[b];

  // waves: WAVES / 2 wave rows x 2 wave columns; wave row wm takes the 16-row sub-tiles
  // wm, wm + WMW, ... (at most NVMAX of them), wave column wn half of the weight columns
  constexpr int WMW = WAVES / 2, NVMAX = (C::BM / 16) / WMW;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so the LDS destinations of the direct loads are scalar (no per-load readfirstlane)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t row_bytes = (int64_t)Kd * M::kElemBytes;
  const int nk = (int)(row_bytes / kPRowBytes) / ksplit;   // stages of this part
  const int64_t kbeg = (int64_t)ksp * nk * kPRowBytes;

  // ---- direct-load sources. Wave w issues token-row loads a = w*LA .. and weight-row loads
  // q = w*LB ..; load a covers block rows [8a, 8a+8): lane -> row 8a + lane/8, chunk slot lane%8,
  // global chunk = slot ^ row%8.
  constexpr int LA = C::kLoadsA / WAVES, LB = C::kLoadsB / WAVES;
  const int lrow = lane / kPChunks;
  const int gchunk = (lane % kPChunks) ^ lrow;
  // token rows: gathered from x (gate/up; x is under 4 GiB, checked by the host) or the block's own
  // rows of h (down)
  const unsigned char* abase = GATE_UP ? A : A + (int64_t)row0 * row_bytes;
  const uint32_t abytes = GATE_UP ? 0xffffffffu : (uint32_t)(rows * row_bytes);
  uint32_t aoff[LA];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    int rr = (wave * LA + q) * kPRowsPerLoad + lrow;   // block row 0..BM-1
    if (rr >= rows) rr = rows - 1;                      // padding rows re-read a valid row
    const int64_t arow = GATE_UP ? (int64_t)(at.sorted_slot[row0 + rr] / topk) : (int64_t)rr;
    aoff[q] = (uint32_t)(arow * row_bytes + kbeg + gchunk * 16);
  }
  // weight tile row br = (wave*LB + q)*8 + lrow; gate/up tiles: rows [0,128) gate, [128,256) up.
  // A wave's LB loads cover 8 LB consecutive tile rows, all in one half. The buffer spans that
  // half of the expert (gate or up rows; down: the expert's matrix), Nout rows (under 4 GiB since
  // H * F < 2^31): a descriptor shared by the waves and workgroups reading the same half ran the
  // prefill gate/up GEMM about 3% faster than one descriptor per wave over just its own rows.
  const int br0 = wave * LB * kPRowsPerLoad;
  const bool up_half = GATE_UP && br0 >= 128;
  const int64_t hrow0 = (int64_t)e * (GATE_UP ? 2 : 1) * Nout + (up_half ? Nout : 0);
  const int64_t wrow0 = (GATE_UP ? 128 * j + (up_half ? br0 - 128 : br0) : 256 * j + br0) + lrow;
  const unsigned char* bbase = W + hrow0 * row_bytes;
  const uint32_t bbytes = (uint32_t)(Nout * row_bytes);
  const uint32_t boff = (uint32_t)(wrow0 * row_bytes + kbeg + gchunk * 16);
  const uint32_t bstep = (uint32_t)(kPRowsPerLoad * row_bytes);   // bytes between consecutive loads

  auto issue_a = [&](int stage) {
    unsigned char* base = aring + (stage % C::AST) * C::kAStageBytes;
    const uint32_t kb = stage * kPRowBytes;
#pragma unroll
    for (int q = 0; q < LA; ++q)
      buffer_load_lds16<0>(abase, abytes, aoff[q], kb,
                           (lds_void_t*)(base + (wave * LA + q) * 1024));
  };
  // weight stages read by one block only stream past L2 (non-temporal); those a group shares keep
  // the default policy, so the group's other blocks find them there
  auto issue_b = [&](int stage) {
    unsigned char* base = bring + (stage % C::BST) * C::kBStageBytes;
    const uint32_t kb = stage * kPRowBytes;
    if (shared_w) {
#pragma unroll
      for (int q = 0; q < LB; ++q)
        buffer_load_lds16<0>(bbase, bbytes, boff + q * bstep, kb,
                             (lds_void_t*)(base + (wave * LB + q) * 1024));
    } else {
#pragma unroll
      for (int q = 0; q < LB; ++q)
        buffer_load_lds16<kCachePolicyNT>(bbase, bbytes, boff + q * bstep, kb,
                                          (lds_void_t*)(base + (wave * LB + q) * 1024));
    }
  };

  floatx4 acc[NVMAX][8];
#pragma unroll
  for (int i = 0; i < NVMAX; ++i)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[i][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Epilogue operands of this tile, staged in LDS after the rings: down: each row's slot id and
  // routing weight (FP8: and its row scale); FP8: the tile's 256 output-channel scales; FP8
  // gate/up: each row's token scale. Their loads go out before the first stage's (the token scale,
  // which needs the slot id, right behind them); they are stored once they have landed.
  static_assert(C::BM <= 64 * WAVES && kPBN <= 64 * WAVES, "one row / column per thread");
  int* const e_slot = reinterpret_cast<int*>(smem + C::kLdsBytes);
  float* const e_w = reinterpret_cast<float*>(smem + C::kLdsBytes + 4 * C::BM);
  float* const e_as = reinterpret_cast<float*>(smem + C::kLdsBytes + 8 * C::BM);
  float* const e_ws = reinterpret_cast<float*>(smem + C::kLdsBytes + 12 * C::BM);
  int v_slot = 0;
  float v_w = 0.f, v_as = 0.f, v_ws = 0.f;
  if constexpr (!GATE_UP) {
    if (tid < rows) {
      v_slot = at.sorted_slot[row0 + tid];
      v_w = at.sorted_w[row0 + tid];
      if constexpr (FP8) v_as = a_scale[row0 + tid];
    }
    if constexpr (FP8)
      if (tid < kPBN) v_ws = w_scale[(int64_t)e * Nout + 256 * j + tid];
  } else if constexpr (FP8) {   // tile columns: 128 gate channels, then the matching up channels
    if (tid < rows) v_slot = at.sorted_slot[row0 + tid];
    if (tid < kPBN)
      v_ws = w_scale[(int64_t)e * 2 * Nout + (tid < 128 ? 0 : Nout - 128) + 128 * j + tid];
  }

  // Issue order: prologue A(0), B(0); iteration kt waits for everything it issued, passes the
  // barrier (every wave's loads of stage kt have landed and every wave is done reading stage
  // kt - 1, whose slots are reused), then issues A(kt+1), B(kt+1) and computes stage kt.
  issue_a(0);
  issue_b(0);
  if constexpr (GATE_UP && FP8)
    if (tid < rows) v_as = a_scale[v_slot / topk];
  if constexpr (!GATE_UP || FP8) {
    if (tid < C::BM) {
      if constexpr (!GATE_UP) {
        e_slot[tid] = v_slot;
        e_w[tid] = v_w;
      }
      if constexpr (FP8) e_as[tid] = v_as;
    }
    if constexpr (FP8)
      if (tid < kPBN) e_ws[tid] = v_ws;
  }

  // fragment byte offsets of this lane inside a 16-row group, per MFMA step of a stage:
  // row r = lane % 16, chunk M::chunk(step, lane / 16, half) (swizzled)
  const int r = lane & 15, g = lane >> 4;
  int frag_off[M::kSteps][M::kReads];
#pragma unroll
  for (int s = 0; s < M::kSteps; ++s)
#pragma unroll
    for (int h = 0; h < M::kReads; ++h)
      frag_off[s][h] = r * kPRowBytes + ((M::chunk(s, g, h) ^ (r & 7)) << 4);

  auto kloop = [&](auto nv_tag) {
    constexpr int NV = decltype(nv_tag)::value;
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_ring_barrier();
      if (kt + 1 < nk) issue_a(kt + 1);
      if (kt + 1 < nk) issue_b(kt + 1);
      const unsigned char* sa = aring + (kt % C::AST) * C::kAStageBytes;
      const unsigned char* sb = bring + (kt % C::BST) * C::kBStageBytes;
      if constexpr (FP8) {
        // FP8 fragments are 8 registers: the token fragments are read once, the weight fragments
        // in two halves of 4, each half followed by its MFMAs, so 160 accumulators and two waves
        // per SIMD fit (254 registers, no spills; reading every token fragment once per half
        // instead measured 4% slower)
        typename M::frag af[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
          af[i] = M::read(sa + (wm + WMW * i) * 16 * kPRowBytes, frag_off[0]);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          typename M::frag bw[4];
#pragma unroll
          for (int nn = 0; nn < 4; ++nn) {
            const int n = 4 * hb + nn;
            const int grp = GATE_UP ? (n < 4 ? 4 * wn + n : 8 + 4 * wn + (n - 4)) : 8 * wn + n;
            bw[nn] = M::read(sb + grp * 16 * kPRowBytes, frag_off[0]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int nn = 0; nn < 4; ++nn)
              acc[i][4 * hb + nn] = M::mma(af[i], bw[nn], acc[i][4 * hb + nn]);
        }
        continue;
      }
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) {
        typename M::frag bw[8], af[NV];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          int grp;   // 16-row group of the weight tile feeding N sub-tile n of this wave
          if constexpr (GATE_UP)
            grp = n < 4 ? 4 * wn + n : 8 + 4 * wn + (n - 4);
          else
            grp = 8 * wn + n;
          bw[n] = M::read(sb + grp * 16 * kPRowBytes, frag_off[s]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)   // 16-row sub-tile wm + WMW i of the block
          af[i] = M::read(sa + (wm + WMW * i) * 16 * kPRowBytes, frag_off[s]);
        __builtin_amdgcn_sched_barrier(0);   // all reads ahead of the MFMA chain
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int n = 0; n < 8; ++n) acc[i][n] = M::mma(af[i], bw[n], acc[i][n]);
      }
    }
  };
  // valid sub-tiles of this wave: mt = wm + WMW i < ceil(rows / 16); four loop bodies
  const int nsub = (rows + 15) >> 4;
  const int nv = nsub > wm ? min(NVMAX, (nsub - wm + WMW - 1) / WMW) : 0;
  static_assert(NVMAX == 5, "loop bodies for 5 sub-tiles per wave");
  if (nv > 4)
    kloop(std::integral_constant<int, 5>{});
  else if (nv > 3)
    kloop(std::integral_constant<int, 4>{});
  else if (nv > 2)
    kloop(std::integral_constant<int, 3>{});
  else
    kloop(std::integral_constant<int, 2>{});

  // ---- epilogue ----
  if constexpr (!GATE_UP || FP8) __syncthreads();   // the staged operands are visible
#pragma unroll
  for (int i = 0; i < NVMAX; ++i) {
    const int mt = wm + WMW * i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = mt * 16 + 4 * g + q;
      if (row >= rows) continue;
      if constexpr (GATE_UP) {
        float sx = 1.f;
        if constexpr (FP8) sx = e_as[row];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int tc = 64 * wn + 16 * n + r, hcol = 128 * j + tc;
          float gv = acc[i][n][q], uv = acc[i][n + 4][q];
          if constexpr (FP8) {
            gv = gv * sx * e_ws[tc];
            uv = uv * sx * e_ws[128 + tc];
          }
          const float h = silu_f32(bf16_round(gv)) * bf16_round(uv);
          reinterpret_cast<uint16_t*>(out)[(int64_t)(row0 + row) * Nout + hcol] =
              (uint16_t)f32_to_bf16_bits(h);
        }
      } else {
        const int slot = e_slot[row];
        const float wgt = e_w[row];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int tc = 128 * wn + 16 * n + r, col = 256 * j + tc;
          float y = acc[i][n][q];
          if constexpr (FP8) y = y * e_as[row] * e_ws[tc];
          reinterpret_cast<float*>(out)[((int64_t)slot * ksplit + ksp) * Nout + col] = wgt * y;
        }
      }
    }
  }
}

}  // namespace beam
