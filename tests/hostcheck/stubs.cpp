// Host-only stand-ins for the sanitizer build of the dispatcher (tests/hostcheck): the few HIP
// runtime calls the dispatcher makes, a gfx950 device that is always "current", and every kernel
// launcher replaced by a check that each buffer the launch would touch lies inside memory the
// driver registered (inputs, outputs, the workspace). Nothing here runs on a GPU; the "device"
// buffers are reserved address ranges that are never dereferenced.
#include "hostcheck.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../routing_grouped_expert_fp32_amd/csrc/common.h"

namespace hostcheck {

namespace {
struct Range {
  uintptr_t lo, hi;
  const char* name;
};
std::vector<Range> g_ranges;
long g_launches = 0;
long g_syncs = 0;
}  // namespace

void register_range(const void* p, size_t bytes, const char* name) {
  g_ranges.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes, name});
}
void clear_ranges() { g_ranges.clear(); }
long launches() { return g_launches; }
long syncs() { return g_syncs; }

// [p, p + bytes) must lie inside one registered range (bytes == 0: only the start is checked).
void need(const char* launcher, const char* what, const void* p, size_t bytes) {
  if (!p) {
    std::fprintf(stderr, "%s: %s is NULL\n", launcher, what);
    std::abort();
  }
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  for (const Range& r : g_ranges)
    if (a >= r.lo && a < r.hi) {
      if (a + bytes > r.hi) {
        std::fprintf(stderr, "%s: %s [%#lx, +%zu) runs %zu bytes past the end of %s\n", launcher,
                     what, (unsigned long)a, bytes, (size_t)(a + bytes - r.hi), r.name);
        std::abort();
      }
      return;
    }
  std::fprintf(stderr, "%s: %s %#lx lies in no registered buffer\n", launcher, what,
               (unsigned long)a);
  std::abort();
}

}  // namespace hostcheck

using hostcheck::need;

// ---- HIP runtime -------------------------------------------------------------------------------
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int) {
  std::memset(p, 0, sizeof(*p));
  std::strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
  p->multiProcessorCount = 256;
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  static char token[64];
  *e = reinterpret_cast<hipEvent_t>(token);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.001f;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) {
  ++hostcheck::g_syncs;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }

// ---- kernel launchers ----------------------------------------------------------------------------
namespace beam {
namespace {
hipError_t launched() {
  ++hostcheck::g_launches;
  return hipSuccess;
}
size_t TKs(const Shape& s) { return (size_t)s.T * (size_t)s.K; }
void need_tables(const char* l, const AlignTables& at, const Shape& s) {
  const size_t n_chunks = (size_t)ceil_div(s.T, kAlignChunk);
  need(l, "chunk_mask", at.chunk_mask, 8 * kAlignWords * n_chunks * (size_t)s.E);
  need(l, "chunk_base", at.chunk_base, 4 * n_chunks * (size_t)s.E);
  need(l, "expert_count", at.expert_count, 4 * (size_t)s.E);
  need(l, "expert_off", at.expert_off, 4 * ((size_t)s.E + 1));
  need(l, "n_blocks", at.n_blocks, 4);
  need(l, "blk_expert", at.blk_expert, 0);
  need(l, "blk_row0", at.blk_row0, 0);
  need(l, "blk_rows", at.blk_rows, 0);
  need(l, "sorted_slot", at.sorted_slot, 4 * TKs(s));
  need(l, "sorted_w", at.sorted_w, 4 * TKs(s));
}
void need_blocks(const char* l, const AlignTables& at, int64_t max_blocks) {
  need(l, "blk_expert", at.blk_expert, 4 * (size_t)max_blocks);
  need(l, "blk_row0", at.blk_row0, 4 * (size_t)max_blocks);
  need(l, "blk_rows", at.blk_rows, 4 * (size_t)max_blocks);
}
}  // namespace

hipError_t launch_router_logits(const void* x, bool x_bf16, const float* w, const float* bias,
                                float2* sb, const Shape& s, hipStream_t) {
  const char* l = "router_logits";
  need(l, "x", x, (size_t)s.T * s.H * (x_bf16 ? 2 : 4));
  need(l, "w_router", w, 4 * (size_t)s.E * s.H);
  need(l, "bias", bias, 4 * (size_t)s.E);
  need(l, "sb", sb, 8 * (size_t)s.T * s.E);
  return launched();
}
hipError_t launch_router_partials(const void* x, bool x_bf16, const float* w, float* part,
                                  const Shape& s, hipStream_t) {
  const char* l = "router_partials";
  need(l, "x", x, (size_t)s.T * s.H * (x_bf16 ? 2 : 4));
  need(l, "w_router", w, 4 * (size_t)s.E * s.H);
  need(l, "part", part, 4 * (size_t)router_partial_chunks(s) * s.T * s.E);
  return launched();
}
hipError_t launch_router_select_partials(const float* part, const float* bias, int32_t* ids,
                                         float* w, const Shape& s, hipStream_t) {
  const char* l = "router_select_partials";
  need(l, "part", part, 4 * (size_t)router_partial_chunks(s) * s.T * s.E);
  need(l, "bias", bias, 4 * (size_t)s.E);
  need(l, "ids", ids, 4 * TKs(s));
  need(l, "w", w, 4 * TKs(s));
  return launched();
}
hipError_t launch_router_select(const float2* sb, int32_t* ids, float* w, const Shape& s,
                                hipStream_t) {
  const char* l = "router_select";
  need(l, "sb", sb, 8 * (size_t)s.T * s.E);
  need(l, "ids", ids, 4 * TKs(s));
  need(l, "w", w, 4 * TKs(s));
  return launched();
}
hipError_t launch_router_split(const float* w, uint16_t* planes, const Shape& s, hipStream_t) {
  const char* l = "router_split";
  need(l, "w_router", w, 4 * (size_t)s.E * s.H);
  need(l, "planes", planes, 6 * (size_t)s.E * s.H);
  return launched();
}
hipError_t launch_router_fused(const void* x, const uint16_t* planes, const float* bias,
                               int32_t* ids, float* w, const Shape& s, hipStream_t) {
  const char* l = "router_fused";
  if (!use_fused_router(s, true)) return hipErrorInvalidValue;
  need(l, "x", x, 2 * (size_t)s.T * s.H);
  need(l, "planes", planes, 6 * (size_t)s.E * s.H);
  need(l, "bias", bias, 4 * (size_t)s.E);
  need(l, "ids", ids, 4 * TKs(s));
  need(l, "w", w, 4 * TKs(s));
  return launched();
}
hipError_t launch_fill_dense_routes(int32_t* ids, float* w, int64_t n, hipStream_t) {
  need("fill_dense_routes", "ids", ids, 4 * (size_t)n);
  need("fill_dense_routes", "w", w, 4 * (size_t)n);
  return launched();
}
hipError_t launch_align(const int32_t* ids, const float* tw, const AlignTables& at,
                        const Shape& s, int, int, int, hipStream_t) {
  need("align", "ids", ids, 4 * TKs(s));
  need("align", "topk_w", tw, 4 * TKs(s));
  need_tables("align", at, s);
  return launched();
}
hipError_t launch_select_align_small(const float* part, const float* bias, int32_t* ids, float* w,
                                     const AlignTables& at, const Shape& s, int, hipStream_t) {
  const char* l = "select_align_small";
  if (!use_fused_select_align(s)) return hipErrorInvalidValue;
  need(l, "part", part, 4 * (size_t)router_partial_chunks(s) * s.T * s.E);
  need(l, "bias", bias, 4 * (size_t)s.E);
  need(l, "ids", ids, 4 * TKs(s));
  need(l, "w", w, 4 * TKs(s));
  need_tables(l, at, s);
  return launched();
}
hipError_t launch_gate_up(const void* x, const void* w_gu, uint16_t* hbuf, const float* x_scale,
                          const float* w_scale, bool fp8, const AlignTables& at, const Shape& s,
                          int64_t max_blocks, bool, hipStream_t) {
  const char* l = "gate_up";
  need(l, "x", x, (size_t)s.T * s.H * (fp8 ? 1 : 2));
  need(l, "w_gate_up", w_gu, 0);
  need(l, "h", hbuf, 2 * TKs(s) * s.F);
  if (fp8) {
    need(l, "x_scale", x_scale, 4 * (size_t)s.T);
    need(l, "w_scale", w_scale, 0);
  }
  need_tables(l, at, s);
  need_blocks(l, at, max_blocks);
  return launched();
}
hipError_t launch_down(const void* h, const void* w_dn, const float* h_scale, const float* w_scale,
                       bool fp8, float* ybuf, const AlignTables& at, const Shape& s,
                       int64_t max_blocks, bool, hipStream_t, int ksplit) {
  const char* l = "down";
  need(l, "h", h, TKs(s) * s.F * (fp8 ? 1 : 2));
  need(l, "w_down", w_dn, 0);
  need(l, "Y", ybuf, 4 * TKs(s) * (size_t)ksplit * s.H);
  if (fp8) {
    need(l, "h_scale", h_scale, 4 * TKs(s));
    need(l, "w_scale", w_scale, 0);
  }
  need_tables(l, at, s);
  need_blocks(l, at, max_blocks);
  return launched();
}
hipError_t launch_gate_up_f32(const float* x, const float* w_gu, float* hbuf, const AlignTables& at,
                              const Shape& s, int64_t max_blocks, hipStream_t) {
  need("gate_up_f32", "x", x, 4 * (size_t)s.T * s.H);
  need("gate_up_f32", "w_gate_up", w_gu, 0);
  need("gate_up_f32", "h", hbuf, 4 * TKs(s) * s.F);
  need_tables("gate_up_f32", at, s);
  need_blocks("gate_up_f32", at, max_blocks);
  return launched();
}
hipError_t launch_down_f32(const float* hbuf, const float* w_dn, const float* tw, float* ybuf,
                           const AlignTables& at, const Shape& s, int64_t max_blocks,
                           hipStream_t) {
  need("down_f32", "h", hbuf, 4 * TKs(s) * s.F);
  need("down_f32", "w_down", w_dn, 0);
  need("down_f32", "topk_w", tw, 4 * TKs(s));
  need("down_f32", "Y", ybuf, 4 * TKs(s) * s.H);
  need_tables("down_f32", at, s);
  need_blocks("down_f32", at, max_blocks);
  return launched();
}
hipError_t launch_quant_rows_fp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* codes,
                                 float* scales, hipStream_t, const int32_t* n_rows) {
  need("quant_rows_fp8", "src", src, 2 * (size_t)rows * cols);
  need("quant_rows_fp8", "codes", codes, (size_t)rows * cols);
  need("quant_rows_fp8", "scales", scales, 4 * (size_t)rows);
  if (n_rows) need("quant_rows_fp8", "n_rows", n_rows, 4);
  return launched();
}
hipError_t launch_convert(const float* src, int64_t n, bool to_fp8, void* dst, hipStream_t) {
  need("convert", "src", src, 4 * (size_t)n);
  need("convert", "dst", dst, (size_t)n * (to_fp8 ? 1 : 2));
  return launched();
}
hipError_t launch_fp8_dot_tiles(const uint8_t* A, const uint8_t* B, const float* C, float* D,
                                int64_t n, hipStream_t) {
  need("fp8_dot_tiles", "a", A, 2048 * (size_t)n);
  need("fp8_dot_tiles", "b", B, 2048 * (size_t)n);
  need("fp8_dot_tiles", "c", C, 1024 * (size_t)n);
  need("fp8_dot_tiles", "d", D, 1024 * (size_t)n);
  return launched();
}
hipError_t scratch_of_current_device(void** out) {
  *out = hostcheck::scratch_range();
  return hipSuccess;
}
hipError_t launch_boundary(const BoundaryArgs& b, const float* Y, int K, const int32_t* ids, int,
                           int, const void* y, bool y_bf16, int64_t T, int H, hipStream_t) {
  const char* l = "boundary";
  const size_t TH = (size_t)T * H;
  need(l, "h", b.h, 2 * TH);
  need(l, "gamma_post", b.gamma_post, 4 * (size_t)H);
  need(l, "gamma_next", b.gamma_next, 4 * (size_t)H);
  need(l, "h_out", b.h_out, 2 * TH);
  need(l, "x_next", b.x_next, 2 * TH);
  if (Y) {
    need(l, "Y", Y, 4 * TH * (size_t)K);
    if (ids) need(l, "ids", ids, 4 * (size_t)T * K);
  } else {
    need(l, "y", y, TH * (y_bf16 ? 2 : 4));
  }
  return launched();
}
hipError_t launch_combine(const float* ybuf, void* out, bool out_bf16, const Shape& s,
                          const int32_t* ids, int, int, hipStream_t) {
  // s.K counts partial rows per token (slots x K-split parts)
  need("combine", "Y", ybuf, 4 * TKs(s) * s.H);
  need("combine", "out", out, (size_t)s.T * s.H * (out_bf16 ? 2 : 4));
  if (ids) need("combine", "ids", ids, 0);
  return launched();
}
}  // namespace beam
