// Internal declarations of the Beam MoE library shared by the host dispatcher and the kernels
// (gfx950 only): shapes, workspace tables, sizes and the kernel launchers. Plain C++ plus the HIP
// runtime API; device-side helpers are in device_common.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace beam {

constexpr int kWave = 64;
constexpr int kAlignChunk = 256;              // tokens per align chunk (one mask bit each)
constexpr int kAlignWords = kAlignChunk / 64; // 64-bit mask words per (chunk, expert)

// ---- routing/align tables carved from the workspace ------------------------------------------
struct AlignTables {
  uint64_t* chunk_mask;   // [n_chunks][E][kAlignWords]  bit j: token kAlignChunk*c+j chose e
  int32_t* chunk_base;    // [n_chunks][E]  rows of expert e in chunks before c
  int32_t* expert_count;  // [E]
  int32_t* expert_off;    // [E+1] exclusive prefix of counts (rows in sorted order)
  int32_t* n_blocks;      // [1]
  int32_t* blk_expert;    // [max_blocks]
  int32_t* blk_row0;      // [max_blocks] first sorted row of the block
  int32_t* blk_rows;      // [max_blocks] rows in the block (1..BM)
  int32_t* sorted_slot;   // [T*K] slot id (t*K+k) of each sorted row
  float* sorted_w;        // [T*K] routing weight of each sorted row (topk_w[sorted_slot[i]])
};


inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sizes shared by the kernels and the host-side dispatch rules (host_rules.cpp), which is plain C++
// so the dispatcher and validation also build without the GPU compiler (sanitizer checks).
constexpr int kSmallBlockRows = 16;      // rows of a moe_align block for the streaming GEMMs
constexpr int kPipeBlockRows = 320;      // ... and for the LDS-tiled GEMMs (bf16 and FP8)
constexpr int kRouterChunk = 256;        // hidden chunk of the partial-logit and one-pass routers
constexpr int kRouterMaxChunks = 32;     // most hidden chunks the partial-logit selection sums
constexpr int kBoundaryMaxHidden = 16 * 4 * 256;   // widest row of the boundary kernel

// Upper bound on the number of row blocks when every expert's rows are split into ceil(c/BM)
// blocks: sum_e ceil(c_e/BM) <= floor(TK/BM) + min(E, TK) + 1.
inline int64_t max_row_blocks(int64_t TK, int64_t E, int64_t BM) {
  int64_t nz = TK < E ? TK : E;
  return TK / BM + nz + 1;
}

}  // namespace beam

// ---- launchers (host side, defined in the .hip files) -------------------------------------------
namespace beam {
struct Shape {
  int64_t T;
  int32_t H, E, G, Gk, K, F;
  float scale;
};

hipError_t launch_router_logits(const void* x, bool x_bf16, const float* w_router,
                                const float* bias, float2* sb, const Shape& s, hipStream_t st);
// Batches of at most kPartialRouteT tokens are routed through partial logits split over 256-wide
// hidden chunks (many workgroups stream W_r; the selection sums the chunks in order); larger ones
// take the one-pass router with bf16 activations (use_fused_router), else the logits kernel and
// the selection. Its time barely grows with T (each workgroup streams all of W_r once), the partial
// path's grows linearly: they cross near 1100 tokens at Beam's shape.
constexpr int64_t kPartialRouteT = 1024;
// batches of at most kSmallAlignT tokens are aligned by one workgroup
constexpr int64_t kSmallAlignT = 64;
int router_partial_chunks(const Shape& s);
bool use_partial_route(const Shape& s);
hipError_t launch_router_partials(const void* x, bool x_bf16, const float* w_router, float* part,
                                  const Shape& s, hipStream_t st);
hipError_t launch_router_select_partials(const float* part, const float* bias, int32_t* ids,
                                         float* w, const Shape& s, hipStream_t st);
hipError_t launch_router_select(const float2* sb, int32_t* ids, float* w, const Shape& s,
                                hipStream_t st);
// bf16 activations past the partial path: the router weights split exactly into three bf16 planes
// (3 E H bf16, in MFMA fragment order; launch_router_split), then logits and selection in one
// launch with no HBM round trip
bool use_fused_router(const Shape& s, bool x_bf16);
hipError_t launch_router_split(const float* w_router, uint16_t* planes, const Shape& s,
                               hipStream_t st);
hipError_t launch_router_fused(const void* x, const uint16_t* planes, const float* bias,
                               int32_t* ids, float* w, const Shape& s, hipStream_t st);
hipError_t launch_fill_dense_routes(int32_t* ids, float* w, int64_t n, hipStream_t st);
hipError_t launch_align(const int32_t* ids, const float* topk_w, const AlignTables& at,
                        const Shape& s, int BM, int e_begin, int e_count, hipStream_t st);
// T <= kFusedSelectT: the selection from partial logits and the align of its routes, one launch
// of one workgroup (a wave per token; larger small batches select over many workgroups first)
constexpr int64_t kFusedSelectT = 16;
inline bool use_fused_select_align(const Shape& s) {
  return s.T <= kFusedSelectT && s.K <= 16 && s.T <= kSmallAlignT && use_partial_route(s);
}
hipError_t launch_select_align_small(const float* part, const float* bias, int32_t* ids, float* w,
                                     const AlignTables& at, const Shape& s, int BM, hipStream_t st);
// bf16 or FP8 experts; FP8 needs the activation scales (per token for x, per sorted row for h)
// and the per-output-channel weight scales.
hipError_t launch_gate_up(const void* x, const void* w_gu, uint16_t* hbuf, const float* x_scale,
                          const float* w_scale, bool fp8, const AlignTables& at, const Shape& s,
                          int64_t max_blocks, bool small, hipStream_t st);
// Each row's routing weight comes from the align tables (sorted_w). ksplit > 1 (tiled blocks only,
// stages of a row divisible by it): the down GEMM's K range is cut into ksplit parts whose partial
// sums go to rows slot * ksplit + part of ybuf.
hipError_t launch_down(const void* h, const void* w_dn, const float* h_scale, const float* w_scale,
                       bool fp8, float* ybuf, const AlignTables& at, const Shape& s,
                       int64_t max_blocks, bool small, hipStream_t st, int ksplit = 1);
// K split (1, 2 or 4) for a tiled down GEMM of `tiles` (block, column tile) workgroups over
// `k_stages` 128-byte stages on a GPU of n_cu compute units.
int down_ksplit(int64_t tiles, int64_t k_stages, int n_cu);
// Column tiles of the tiled down GEMM (output columns per workgroup: 256).
constexpr int kPipeDownCols = 256;
hipError_t launch_gate_up_f32(const float* x, const float* w_gu, float* hbuf,
                              const AlignTables& at, const Shape& s, int64_t max_blocks,
                              hipStream_t st);
hipError_t launch_down_f32(const float* hbuf, const float* w_dn, const float* topk_w, float* ybuf,
                           const AlignTables& at, const Shape& s, int64_t max_blocks,
                           hipStream_t st);
// n_rows (device, nullable): rows at or past *n_rows are skipped
hipError_t launch_quant_rows_fp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                 float* scales, hipStream_t st, const int32_t* n_rows = nullptr);
hipError_t launch_convert(const float* src, int64_t n, bool to_fp8, void* dst, hipStream_t st);
hipError_t launch_fp8_dot_tiles(const uint8_t* A, const uint8_t* B, const float* C, float* D,
                                int64_t n, hipStream_t st);
int small_block_rows();
int tiled_block_rows(bool fp8);   // rows per block of the tiled GEMMs
// Device address of this GPU's 64 MiB workspace array of the no-allocation entry point (scratch.hip),
// looked up once per device; hipSuccess or the lookup's error.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_of_current_device(void** out);
// post-norm -> depth-scaled residual -> next pre-norm (boundary.hip)
struct BoundaryArgs {
  const uint16_t* h;         // [T][H] bf16 residual stream in
  const float* gamma_post;   // [H]
  const float* gamma_next;   // [H]
  uint16_t* h_out;           // [T][H] bf16 residual stream out (may be h)
  uint16_t* x_next;          // [T][H] bf16 normalised input of the next sublayer
  float alpha, beta, eps;    // sqrt((n-1)/n), 1/sqrt(n), RMSNorm epsilon
};
int boundary_max_hidden();
// Y != nullptr: y = sum of the K slot rows of Y (only ids in [e_begin, e_end) when ids != nullptr);
// otherwise y = the [T][H] fp32 or bf16 array `y`
hipError_t launch_boundary(const BoundaryArgs& b, const float* Y, int K, const int32_t* ids,
                           int e_begin, int e_end, const void* y, bool y_bf16, int64_t T, int H,
                           hipStream_t st);
hipError_t launch_combine(const float* ybuf, void* out, bool out_bf16, const Shape& s,
                          const int32_t* ids, int e_begin, int e_end, hipStream_t st);
}  // namespace beam
