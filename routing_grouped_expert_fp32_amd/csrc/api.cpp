// C ABI of the Beam MoE library: argument validation, workspace carving, kernel dispatch.
// Declarations, argument meanings and error behaviour: include/beam_moe.h.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <algorithm>
#include <vector>

#include "../../include/beam_moe.h"
#include "common.h"

namespace {

using beam::ceil_div;

constexpr int kMaxDevices = 64;
constexpr int kNumStages = 8;
const char* kStageNames[kNumStages] = {"router_logits", "router_select", "moe_align",
                                       "quant_x_fp8",   "gate_up",       "quant_h_fp8",
                                       "down",          "combine"};

size_t al256(size_t b) { return (b + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_bytes(int32_t dt) {
  switch (dt) {
    case BEAM_F32: return 4;
    case BEAM_BF16: return 2;
    case BEAM_FP8_E4M3: return 1;
    default: return 0;
  }
}

// Block rows of moe_align for this call: small decode-like batches stream weights through 16-row
// blocks; larger ones use the LDS-tiled kernels (320-row blocks, bf16 and FP8). FP32 experts use
// 16-row blocks.
bool use_small_blocks(const beam_moe_cfg& c, int64_t T) {
  return c.w_dtype == BEAM_F32 || T * c.topk <= 4 * (int64_t)c.n_experts;
}
int block_rows(const beam_moe_cfg& c, int64_t T) {
  return use_small_blocks(c, T) ? beam::small_block_rows()
                                : beam::tiled_block_rows(c.w_dtype == BEAM_FP8_E4M3);
}

struct Layout {
  size_t sb = 0, ids = 0, w = 0, chunk_mask = 0, chunk_base = 0, expert_count = 0, expert_off = 0,
         n_blocks = 0, blk_expert = 0, blk_row0 = 0, blk_rows = 0, sorted = 0, sorted_w = 0, hbuf = 0,
         ybuf = 0, xq = 0, xs = 0, hq = 0, hs = 0, total = 0;
  int64_t max_blocks = 0;
  int bm = 0;
};

// ybuf_parts > 1: room for the partial sums of a K-split down GEMM (dense layer)
Layout make_layout(const beam_moe_cfg& c, int64_t T, bool full, int ybuf_parts = 1) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al256(bytes);
    return o;
  };
  const int64_t E = c.n_experts, K = c.topk, TK = T * K;
  // Router scratch: the partial logits [H/256][T][E] (partial path), the router weights split into
  // three bf16 planes, 3 E H values (one-pass router), or (s, b) pairs [T][E]. In a forward it
  // shares the region of the expert outputs, which are written only after the routing.
  const beam::Shape s{T, c.hidden, c.n_experts, c.n_groups, c.topk_groups, c.topk, c.d_ff,
                      c.routed_scale};
  size_t route_bytes;
  if (beam::use_partial_route(s))
    route_bytes = sizeof(float) * (size_t)beam::router_partial_chunks(s) * (size_t)(T * E);
  else if (beam::use_fused_router(s, c.x_dtype == BEAM_BF16))
    route_bytes = 6 * (size_t)E * (size_t)c.hidden;
  else
    route_bytes = sizeof(float) * (size_t)(2 * T * E);
  if (!full) L.sb = take(route_bytes);
  if (full) {
    const int64_t n_chunks = ceil_div(T, beam::kAlignChunk);
    L.bm = block_rows(c, T);
    L.max_blocks = beam::max_row_blocks(TK, E, L.bm);
    L.ids = take(sizeof(int32_t) * (size_t)TK);
    L.w = take(sizeof(float) * (size_t)TK);
    L.chunk_mask = take(sizeof(uint64_t) * beam::kAlignWords * (size_t)(n_chunks * E));
    L.chunk_base = take(sizeof(int32_t) * (size_t)(n_chunks * E));
    L.expert_count = take(sizeof(int32_t) * (size_t)E);
    L.expert_off = take(sizeof(int32_t) * (size_t)(E + 1));
    L.n_blocks = take(sizeof(int32_t));
    L.blk_expert = take(sizeof(int32_t) * (size_t)L.max_blocks);
    L.blk_row0 = take(sizeof(int32_t) * (size_t)L.max_blocks);
    L.blk_rows = take(sizeof(int32_t) * (size_t)L.max_blocks);
    L.sorted = take(sizeof(int32_t) * (size_t)TK);
    L.sorted_w = take(sizeof(float) * (size_t)TK);
    const size_t hel = c.w_dtype == BEAM_F32 ? 4 : 2;
    L.hbuf = take(hel * (size_t)TK * (size_t)c.d_ff);
    if (c.w_dtype == BEAM_FP8_E4M3) {
      L.xq = take((size_t)T * (size_t)c.hidden);
      L.xs = take(sizeof(float) * (size_t)T);
      L.hq = take((size_t)TK * (size_t)c.d_ff);
      L.hs = take(sizeof(float) * (size_t)TK);
    }
    // last, so the offsets above do not depend on the number of partial rows per slot
    L.ybuf = take(std::max(sizeof(float) * (size_t)TK * (size_t)ybuf_parts * (size_t)c.hidden,
                           route_bytes));
    L.sb = L.ybuf;
  }
  L.total = off;
  return L;
}

beam_status_t check_cfg(const beam_moe_cfg* c, bool experts) {
  if (!c) return BEAM_ERR_NULL;
  if (c->hidden <= 0 || c->n_experts <= 0 || c->n_groups <= 0 || c->topk_groups <= 0 ||
      c->topk <= 0 || (experts && c->d_ff <= 0))
    return BEAM_ERR_SHAPE;
  if (c->n_experts % c->n_groups != 0 || c->topk_groups > c->n_groups ||
      c->topk > c->topk_groups * (c->n_experts / c->n_groups))
    return BEAM_ERR_SHAPE;
  if (!(std::isfinite(c->routed_scale) && c->routed_scale > 0.f)) return BEAM_ERR_SHAPE;
  const bool xd = c->x_dtype == BEAM_F32 || c->x_dtype == BEAM_BF16;
  const bool wd = c->w_dtype == BEAM_F32 || c->w_dtype == BEAM_BF16 || c->w_dtype == BEAM_FP8_E4M3;
  const bool od = c->out_dtype == BEAM_F32 || c->out_dtype == BEAM_BF16;
  if (!xd || !wd || !od) return BEAM_ERR_DTYPE;
  if ((c->x_dtype == BEAM_F32) != (c->w_dtype == BEAM_F32)) return BEAM_ERR_DTYPE;
  // limits of this library version
  if (c->hidden % 256 != 0 || c->n_experts > 256 || c->n_experts % 16 != 0 ||
      (c->n_experts > 64 && c->n_experts % 64 != 0) || c->n_groups > 64 || c->topk > 16)
    return BEAM_ERR_UNSUPPORTED;
  if (experts) {
    if (c->d_ff % 256 != 0 || (int64_t)c->hidden * c->d_ff >= (int64_t(1) << 31))
      return BEAM_ERR_UNSUPPORTED;
  }
  return BEAM_OK;
}

// bf16 activations under 4 GiB: the tiled expert GEMM gathers token rows with 32-bit offsets
bool x_fits_offsets(int64_t T, int64_t hidden) {
  return (uint64_t)T * (uint64_t)hidden < (uint64_t(1) << 31);
}

beam_status_t check_T(const beam_moe_cfg* c, int64_t T, bool experts) {
  if (T < 0) return BEAM_ERR_SHAPE;
  if (T * c->topk >= (int64_t(1) << 31) || T >= (int64_t(1) << 31)) return BEAM_ERR_UNSUPPORTED;
  if (experts && c->x_dtype == BEAM_BF16 && !x_fits_offsets(T, c->hidden))
    return BEAM_ERR_UNSUPPORTED;
  return BEAM_OK;
}

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + bytes};
}
bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// every output must be disjoint from every input and every other output
bool any_alias(const std::vector<Range>& ins, const std::vector<Range>& outs) {
  for (size_t i = 0; i < outs.size(); ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (const auto& r : ins)
      if (r.lo != r.hi && overlap(outs[i], r)) return true;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (outs[j].lo != outs[j].hi && overlap(outs[i], outs[j])) return true;
  }
  return false;
}

int g_cus[kMaxDevices];   // compute units per device, cached by check_device

beam_status_t check_device() {
  static int arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BEAM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BEAM_ERR_DEVICE;
    arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev] = prop.multiProcessorCount;
  }
  return arch_ok[dev] == 1 ? BEAM_OK : BEAM_ERR_DEVICE;
}

// compute units of the current device (after a successful check_device)
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  return g_cus[dev] > 0 ? g_cus[dev] : 256;
}

// ---- stage timing ------------------------------------------------------------------------------
struct TimingRec {
  int stage;
  hipEvent_t a, b;
};
std::vector<TimingRec> g_recs;
bool g_timing = false;
uint32_t g_timing_mask = ~0u;

struct StageTimer {
  int stage;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  StageTimer(int s, hipStream_t stream) : stage(s), st(stream) {
    if (!g_timing || !((g_timing_mask >> stage) & 1u)) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      a = b = nullptr;
      return;
    }
    if (hipEventRecord(a, st) != hipSuccess) release();
  }
  ~StageTimer() {
    if (!a) return;
    if (hipEventRecord(b, st) != hipSuccess) {
      release();
      return;
    }
    g_recs.push_back({stage, a, b});
  }
  void release() {   // a failed record: drop this stage's events (timing is best effort)
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    a = b = nullptr;
  }
};

// BEAM_MOE_SYNC_CHECK set to anything but "0" (read once): every launch is followed by a
// synchronisation of its stream, and a kernel that failed is reported (stderr, naming the stage)
// as BEAM_ERR_LAUNCH from the call that launched it. A debugging aid: it serialises the host with
// the GPU and must not be used under stream capture.
bool sync_check() {
  static const bool on = [] {
    const char* v = std::getenv("BEAM_MOE_SYNC_CHECK");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

beam_status_t launched(hipError_t err, hipStream_t st, const char* what) {
  if (err == hipSuccess && sync_check()) err = hipStreamSynchronize(st);
  if (err == hipSuccess) return BEAM_OK;
  std::fprintf(stderr, "beam_moe: %s failed: %s\n", what, hipGetErrorString(err));
  return BEAM_ERR_LAUNCH;
}

#define LAUNCH(stage, expr)                                                            \
  do {                                                                                 \
    StageTimer timer_((stage), st);                                                    \
    if (launched((expr), st, kStageNames[(stage)]) != BEAM_OK) return BEAM_ERR_LAUNCH; \
  } while (0)

beam::Shape shape_of(const beam_moe_cfg& c, int64_t T) {
  return beam::Shape{T, c.hidden, c.n_experts, c.n_groups, c.topk_groups, c.topk, c.d_ff,
                     c.routed_scale};
}

beam::AlignTables align_tables(const Layout& L, char* ws) {
  beam::AlignTables at;
  at.chunk_mask = reinterpret_cast<uint64_t*>(ws + L.chunk_mask);
  at.chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  at.expert_count = reinterpret_cast<int32_t*>(ws + L.expert_count);
  at.expert_off = reinterpret_cast<int32_t*>(ws + L.expert_off);
  at.n_blocks = reinterpret_cast<int32_t*>(ws + L.n_blocks);
  at.blk_expert = reinterpret_cast<int32_t*>(ws + L.blk_expert);
  at.blk_row0 = reinterpret_cast<int32_t*>(ws + L.blk_row0);
  at.blk_rows = reinterpret_cast<int32_t*>(ws + L.blk_rows);
  at.sorted_slot = reinterpret_cast<int32_t*>(ws + L.sorted);
  at.sorted_w = reinterpret_cast<float*>(ws + L.sorted_w);
  return at;
}

// Steps after routing: align, (FP8 quantisation,) gate/up, down, combine, over the experts
// [e_begin, e_begin + e_count) whose weights start at w_gate_up / w_down (and the FP8 scales).
// `filter` makes the combine skip slots routed outside that range.
beam_status_t run_experts(const beam_moe_cfg& c, int64_t T, const Layout& L, char* ws,
                          const int32_t* ids, const float* tw, const void* x,
                          const void* w_gate_up, const void* w_down,
                          const float* w_gate_up_scale, const float* w_down_scale, void* out,
                          int e_begin, int e_count, bool filter, hipStream_t st,
                          const beam::BoundaryArgs* bnd = nullptr, int ksplit = 1,
                          bool aligned = false) {
  const beam::AlignTables at = align_tables(L, ws);
  float* ybuf = reinterpret_cast<float*>(ws + L.ybuf);
  const beam::Shape s = shape_of(c, T);
  const bool small = use_small_blocks(c, T);
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;

  if (e_count > 0) {
    if (!aligned) LAUNCH(2, beam::launch_align(ids, tw, at, s, L.bm, e_begin, e_count, st));
    if (c.w_dtype == BEAM_F32) {
      float* hbuf = reinterpret_cast<float*>(ws + L.hbuf);
      LAUNCH(4, beam::launch_gate_up_f32(reinterpret_cast<const float*>(x),
                                         reinterpret_cast<const float*>(w_gate_up), hbuf, at, s,
                                         L.max_blocks, st));
      LAUNCH(6, beam::launch_down_f32(hbuf, reinterpret_cast<const float*>(w_down), tw, ybuf, at,
                                      s, L.max_blocks, st));
    } else if (!fp8) {
      uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + L.hbuf);
      LAUNCH(4, beam::launch_gate_up(x, w_gate_up, hbuf, nullptr, nullptr, false, at, s,
                                     L.max_blocks, small, st));
      LAUNCH(6, beam::launch_down(hbuf, w_down, nullptr, nullptr, false, ybuf, at, s,
                                  L.max_blocks, small, st, ksplit));
    } else {
      uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + L.hbuf);
      uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
      float* xs = reinterpret_cast<float*>(ws + L.xs);
      uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
      float* hs = reinterpret_cast<float*>(ws + L.hs);
      LAUNCH(3, beam::launch_quant_rows_fp8(reinterpret_cast<const uint16_t*>(x), T, c.hidden, xq,
                                            xs, st));
      LAUNCH(4, beam::launch_gate_up(xq, w_gate_up, hbuf, xs, w_gate_up_scale, true, at, s,
                                     L.max_blocks, small, st));
      // a routed call's sorted rows are its local slots only: quantise those (count on the device)
      LAUNCH(5, beam::launch_quant_rows_fp8(hbuf, T * c.topk, c.d_ff, hq, hs, st,
                                            filter ? at.expert_off + e_count : nullptr));
      LAUNCH(6, beam::launch_down(hq, w_down, hs, w_down_scale, true, ybuf, at, s,
                                  L.max_blocks, small, st, ksplit));
    }
  }
  if (bnd) {   // combine fused into the post-MoE boundary
    LAUNCH(7, beam::launch_boundary(*bnd, ybuf, c.topk, filter ? ids : nullptr, e_begin,
                                    e_begin + e_count, nullptr, false, T, c.hidden, st));
    return BEAM_OK;
  }
  beam::Shape sc = s;   // a K-split down leaves ksplit partial rows per slot, summed in order
  sc.K = s.K * ksplit;
  LAUNCH(7, beam::launch_combine(ybuf, out, c.out_dtype == BEAM_BF16, sc, filter ? ids : nullptr,
                                 e_begin, e_begin + e_count, st));
  return BEAM_OK;
}

// Routing of a batch past the partial-logit path: bf16 activations take the one-pass router
// (weight split, then logits and selection in one launch), FP32 ones the logits kernel and then the
// selection. `scratch` is the router scratch region of the workspace.
beam_status_t route_large(const void* x, bool x_bf16, const float* w_router, const float* bias,
                          char* scratch, int32_t* ids, float* tw, const beam::Shape& s,
                          hipStream_t st) {
  if (beam::use_fused_router(s, x_bf16)) {
    uint16_t* planes = reinterpret_cast<uint16_t*>(scratch);
    LAUNCH(0, beam::launch_router_split(w_router, planes, s, st));
    LAUNCH(0, beam::launch_router_fused(x, planes, bias, ids, tw, s, st));
    return BEAM_OK;
  }
  float2* sb = reinterpret_cast<float2*>(scratch);
  LAUNCH(0, beam::launch_router_logits(x, x_bf16, w_router, bias, sb, s, st));
  LAUNCH(1, beam::launch_router_select(sb, ids, tw, s, st));
  return BEAM_OK;
}

// Boundary arguments: validation common to both boundary entry points.
beam_status_t make_boundary(const void* h, const float* gamma_post, const float* gamma_next,
                            void* h_out, void* x_next, int32_t hidden, int32_t depth_n, float eps,
                            beam::BoundaryArgs& b) {
  if (depth_n < 1 || !(std::isfinite(eps) && eps >= 0.f)) return BEAM_ERR_SHAPE;
  if (hidden > beam::boundary_max_hidden()) return BEAM_ERR_UNSUPPORTED;
  if (!h || !gamma_post || !gamma_next || !h_out || !x_next) return BEAM_ERR_NULL;
  if (!aligned16(h) || !aligned16(gamma_post) || !aligned16(gamma_next) || !aligned16(h_out) ||
      !aligned16(x_next))
    return BEAM_ERR_ALIGN;
  const double n = depth_n;
  b.h = reinterpret_cast<const uint16_t*>(h);
  b.gamma_post = gamma_post;
  b.gamma_next = gamma_next;
  b.h_out = reinterpret_cast<uint16_t*>(h_out);
  b.x_next = reinterpret_cast<uint16_t*>(x_next);
  b.alpha = (float)std::sqrt((n - 1.0) / n);
  b.beta = (float)(1.0 / std::sqrt(n));
  b.eps = eps;
  return BEAM_OK;
}

// Alias rule of the boundary outputs: h_out may be h itself (in place) but must not overlap any
// other buffer; x_next must not overlap anything.
bool boundary_alias(const std::vector<Range>& ins_except_h, const Range& h, const Range& h_out,
                    const Range& x_next, const std::vector<Range>& other_outs) {
  std::vector<Range> outs = other_outs;
  outs.push_back(x_next);
  if (!(h_out.lo == h.lo && h_out.hi == h.hi)) {
    outs.push_back(h_out);
    std::vector<Range> ins = ins_except_h;
    ins.push_back(h);
    return any_alias(ins, outs);
  }
  // in place: h (= h_out) is both; it must still be disjoint from every other buffer
  std::vector<Range> ins = ins_except_h;
  outs.push_back(h_out);
  return any_alias(ins, outs);
}

// A dense SwiGLU layer as a one-expert block: E = G = Gk = K = 1, weight 1.
beam_moe_cfg dense_cfg(int32_t hidden, int32_t d_ff, int32_t w_dtype, int32_t out_dtype) {
  return beam_moe_cfg{hidden, 1, 1, 1, 1, d_ff, 1.0f, BEAM_BF16, w_dtype, out_dtype};
}

beam_status_t check_dense(int32_t hidden, int32_t d_ff, int32_t w_dtype, int32_t out_dtype,
                          int64_t T) {
  if (hidden <= 0 || d_ff <= 0 || T < 0) return BEAM_ERR_SHAPE;
  if (w_dtype != BEAM_BF16 && w_dtype != BEAM_FP8_E4M3) return BEAM_ERR_DTYPE;
  if (out_dtype != BEAM_F32 && out_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;
  if (hidden % 256 != 0 || d_ff % 256 != 0 || (int64_t)hidden * d_ff >= (int64_t(1) << 31) ||
      T >= (int64_t(1) << 31) || !x_fits_offsets(T, hidden))
    return BEAM_ERR_UNSUPPORTED;
  return BEAM_OK;
}

// Largest K split the dense down GEMM may take (tiled blocks; parts of at least 16 stages). The
// workspace holds that many partial rows per token, so its size does not depend on the device.
int dense_ksplit_max(const beam_moe_cfg& c, int64_t T) {
  if (use_small_blocks(c, T)) return 1;
  const int64_t k_stages = (int64_t)c.d_ff * dtype_bytes(c.w_dtype) / 128;
  int m = 1;
  for (int ks = 2; ks <= 4; ks *= 2)
    if (k_stages % ks == 0 && k_stages / ks >= 16) m = ks;
  return m;
}

// beam_moe_forward on a given workspace (also the no-allocation entry point's body).
beam_status_t forward_impl(const void* x, const float* w_router, const float* bias,
                           const void* w_gate_up, const void* w_down, void* out, int64_t T,
                           const beam_moe_cfg* cfg, const float* w_gate_up_scale,
                           const float* w_down_scale, int32_t* topk_ids_out, float* topk_w_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  beam_status_t rc = check_cfg(cfg, true);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, true)) != BEAM_OK) return rc;
  const beam_moe_cfg& c = *cfg;
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;
  if (!fp8 && (w_gate_up_scale || w_down_scale)) return BEAM_ERR_DTYPE;
  if (T == 0) return BEAM_OK;
  if (!x || !w_router || !bias || !w_gate_up || !w_down || !out || !workspace) return BEAM_ERR_NULL;
  if (fp8 && (!w_gate_up_scale || !w_down_scale)) return BEAM_ERR_NULL;
  const void* ptrs[] = {x, w_router, bias, w_gate_up, w_down, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BEAM_ERR_ALIGN;
  if ((topk_ids_out && !aligned16(topk_ids_out)) || (topk_w_out && !aligned16(topk_w_out)) ||
      (w_gate_up_scale && !aligned16(w_gate_up_scale)) || (w_down_scale && !aligned16(w_down_scale)))
    return BEAM_ERR_ALIGN;
  const Layout L = make_layout(c, T, true);
  if (L.max_blocks > 65535) return BEAM_ERR_UNSUPPORTED;   // grid.y bound of the GEMM launches
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;

  const size_t H = c.hidden, E = c.n_experts, F = c.d_ff, TK = (size_t)(T * c.topk);
  const size_t wb = dtype_bytes(c.w_dtype);
  std::vector<Range> ins = {rng(x, (size_t)T * H * dtype_bytes(c.x_dtype)),
                            rng(w_router, sizeof(float) * E * H), rng(bias, sizeof(float) * E),
                            rng(w_gate_up, wb * E * 2 * F * H), rng(w_down, wb * E * H * F)};
  if (fp8) {
    ins.push_back(rng(w_gate_up_scale, sizeof(float) * E * 2 * F));
    ins.push_back(rng(w_down_scale, sizeof(float) * E * H));
  }
  std::vector<Range> outs = {rng(out, (size_t)T * H * dtype_bytes(c.out_dtype)),
                             rng(workspace, L.total)};
  if (topk_ids_out) outs.push_back(rng(topk_ids_out, sizeof(int32_t) * TK));
  if (topk_w_out) outs.push_back(rng(topk_w_out, sizeof(float) * TK));
  if (any_alias(ins, outs)) return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* tw = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  const beam::Shape s = shape_of(c, T);
  if (beam::use_partial_route(s)) {   // partial logits, selection summing them
    float* part = reinterpret_cast<float*>(ws + L.sb);
    LAUNCH(0, beam::launch_router_partials(x, c.x_dtype == BEAM_BF16, w_router, part, s, st));
    if (beam::use_fused_select_align(s)) {   // the selection and the align in one launch
      LAUNCH(1, beam::launch_select_align_small(part, bias, ids, tw, align_tables(L, ws), s, L.bm,
                                                st));
      return run_experts(c, T, L, ws, ids, tw, x, w_gate_up, w_down, w_gate_up_scale,
                         w_down_scale, out, 0, c.n_experts, false, st, nullptr, 1, true);
    }
    LAUNCH(1, beam::launch_router_select_partials(part, bias, ids, tw, s, st));
  } else if ((rc = route_large(x, c.x_dtype == BEAM_BF16, w_router, bias, ws + L.sb, ids, tw, s,
                               st)) != BEAM_OK) {
    return rc;
  }
  return run_experts(c, T, L, ws, ids, tw, x, w_gate_up, w_down, w_gate_up_scale, w_down_scale,
                     out, 0, c.n_experts, false, st);
}

// Offset and size of one inspectable array of a forward's workspace (beam_moe_workspace_region).
beam_status_t region_of(const beam_moe_cfg& c, const Layout& L, int64_t T, int y_parts,
                        int32_t region, size_t* offset, size_t* bytes) {
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;
  const size_t TK = (size_t)(T * c.topk), F = c.d_ff, H = c.hidden;
  switch (region) {
    case BEAM_WS_EXPERT_OFF: *offset = L.expert_off; *bytes = 4 * (size_t)(c.n_experts + 1); break;
    case BEAM_WS_SORTED_SLOT: *offset = L.sorted; *bytes = 4 * TK; break;
    case BEAM_WS_H: *offset = L.hbuf; *bytes = (c.w_dtype == BEAM_F32 ? 4 : 2) * TK * F; break;
    case BEAM_WS_Y: *offset = L.ybuf; *bytes = 4 * TK * (size_t)y_parts * H; break;
    case BEAM_WS_HQ:
    case BEAM_WS_HS:
    case BEAM_WS_XQ:
    case BEAM_WS_XS:
      if (!fp8) return BEAM_ERR_UNSUPPORTED;
      if (region == BEAM_WS_HQ) { *offset = L.hq; *bytes = TK * F; }
      if (region == BEAM_WS_HS) { *offset = L.hs; *bytes = 4 * TK; }
      if (region == BEAM_WS_XQ) { *offset = L.xq; *bytes = (size_t)T * H; }
      if (region == BEAM_WS_XS) { *offset = L.xs; *bytes = 4 * (size_t)T; }
      break;
    default: return BEAM_ERR_UNSUPPORTED;
  }
  return BEAM_OK;
}

}  // namespace

extern "C" {

const char* beam_status_string(beam_status_t s) {
  switch (s) {
    case BEAM_OK: return "ok";
    case BEAM_ERR_NULL: return "null pointer";
    case BEAM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case BEAM_ERR_SHAPE: return "inconsistent shape";
    case BEAM_ERR_DTYPE: return "unsupported dtype combination";
    case BEAM_ERR_UNSUPPORTED: return "shape or dtype not supported by this library version";
    case BEAM_ERR_WORKSPACE: return "workspace missing or too small";
    case BEAM_ERR_ALIAS: return "output overlaps another buffer";
    case BEAM_ERR_LAUNCH: return "kernel launch failed";
    case BEAM_ERR_DEVICE: return "no gfx950 device current";
    default: return "unknown status";
  }
}

int32_t beam_moe_version(void) { return 100; }

beam_status_t beam_moe_workspace_region(const beam_moe_cfg* cfg, int64_t T, int32_t region,
                                        size_t* offset, size_t* bytes) {
  beam_status_t rc = check_cfg(cfg, true);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, true)) != BEAM_OK) return rc;
  if (!offset || !bytes) return BEAM_ERR_NULL;
  return region_of(*cfg, make_layout(*cfg, T, true), T, 1, region, offset, bytes);
}

beam_status_t beam_dense_mlp_workspace_region(int32_t hidden, int32_t d_ff, int32_t w_dtype,
                                              int64_t T, int32_t region, size_t* offset,
                                              size_t* bytes) {
  beam_status_t rc = check_dense(hidden, d_ff, w_dtype, BEAM_F32, T);
  if (rc != BEAM_OK) return rc;
  if (!offset || !bytes) return BEAM_ERR_NULL;
  const beam_moe_cfg c = dense_cfg(hidden, d_ff, w_dtype, BEAM_F32);
  const int parts = dense_ksplit_max(c, T);
  return region_of(c, make_layout(c, T, true, parts), T, parts, region, offset, bytes);
}

size_t beam_moe_route_workspace_bytes(const beam_moe_cfg* cfg, int64_t T) {
  if (check_cfg(cfg, false) != BEAM_OK || T < 0) return 0;
  return make_layout(*cfg, T, false).total;
}

size_t beam_moe_workspace_bytes(const beam_moe_cfg* cfg, int64_t T) {
  if (check_cfg(cfg, true) != BEAM_OK || T < 0) return 0;
  return make_layout(*cfg, T, true).total;
}

beam_status_t beam_moe_route(const void* x, const float* w_router, const float* bias,
                             int32_t* topk_ids, float* topk_w, int64_t T,
                             const beam_moe_cfg* cfg, void* workspace, size_t workspace_bytes,
                             void* stream) {
  beam_status_t rc = check_cfg(cfg, false);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, false)) != BEAM_OK) return rc;
  if (T == 0) return BEAM_OK;
  const beam_moe_cfg& c = *cfg;
  if (!x || !w_router || !bias || !topk_ids || !topk_w || !workspace) return BEAM_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(bias) || !aligned16(topk_ids) ||
      !aligned16(topk_w) || !aligned16(workspace))
    return BEAM_ERR_ALIGN;
  const Layout L = make_layout(c, T, false);
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;
  const size_t TK = (size_t)(T * c.topk);
  const std::vector<Range> ins = {rng(x, (size_t)T * c.hidden * dtype_bytes(c.x_dtype)),
                                  rng(w_router, sizeof(float) * c.n_experts * c.hidden),
                                  rng(bias, sizeof(float) * c.n_experts)};
  const std::vector<Range> outs = {rng(topk_ids, sizeof(int32_t) * TK),
                                   rng(topk_w, sizeof(float) * TK), rng(workspace, L.total)};
  if (any_alias(ins, outs)) return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const beam::Shape s = shape_of(c, T);
  if (beam::use_partial_route(s)) {
    float* part = reinterpret_cast<float*>(ws + L.sb);
    LAUNCH(0, beam::launch_router_partials(x, c.x_dtype == BEAM_BF16, w_router, part, s, st));
    LAUNCH(1, beam::launch_router_select_partials(part, bias, topk_ids, topk_w, s, st));
    return BEAM_OK;
  }
  return route_large(x, c.x_dtype == BEAM_BF16, w_router, bias, ws + L.sb, topk_ids, topk_w, s,
                     st);
}

beam_status_t beam_moe_forward(const void* x, const float* w_router, const float* bias,
                               const void* w_gate_up, const void* w_down, void* out, int64_t T,
                               const beam_moe_cfg* cfg, const float* w_gate_up_scale,
                               const float* w_down_scale, int32_t* topk_ids_out,
                               float* topk_w_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return forward_impl(x, w_router, bias, w_gate_up, w_down, out, T, cfg, w_gate_up_scale,
                      w_down_scale, topk_ids_out, topk_w_out, workspace, workspace_bytes, stream);
}

beam_status_t beam_moe_forward_noalloc(const void* x, const float* w_router, const float* bias,
                                       const void* w_gate_up, const void* w_down, void* out,
                                       int64_t T, const beam_moe_cfg* cfg,
                                       const float* w_gate_up_scale, const float* w_down_scale,
                                       int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  beam_status_t rc = check_cfg(cfg, true);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, true)) != BEAM_OK) return rc;
  if (T == 0) return BEAM_OK;
  if (make_layout(*cfg, T, true).total > beam::kScratchBytes) return BEAM_ERR_WORKSPACE;
  if ((rc = check_device()) != BEAM_OK) return rc;
  void* scratch_ptr = nullptr;
  if (beam::scratch_of_current_device(&scratch_ptr) != hipSuccess) return BEAM_ERR_DEVICE;
  return forward_impl(x, w_router, bias, w_gate_up, w_down, out, T, cfg, w_gate_up_scale,
                      w_down_scale, topk_ids_out, topk_w_out, scratch_ptr, beam::kScratchBytes,
                      stream);
}

beam_status_t beam_residual_boundary(const void* y, int32_t y_dtype, const void* h,
                                     const float* gamma_post, const float* gamma_next,
                                     void* h_out, void* x_next, int64_t T, int32_t hidden,
                                     int32_t depth_n, float eps, void* stream) {
  if (T < 0 || hidden <= 0) return BEAM_ERR_SHAPE;
  if (y_dtype != BEAM_F32 && y_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;
  if (hidden % 256 != 0 || T >= (int64_t(1) << 31)) return BEAM_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_OK;
  beam::BoundaryArgs b;
  beam_status_t rc = make_boundary(h, gamma_post, gamma_next, h_out, x_next, hidden, depth_n, eps,
                                   b);
  if (rc != BEAM_OK) return rc;
  if (!y) return BEAM_ERR_NULL;
  if (!aligned16(y)) return BEAM_ERR_ALIGN;
  const size_t TH = (size_t)T * hidden;
  const std::vector<Range> ins = {rng(y, TH * dtype_bytes(y_dtype)),
                                  rng(gamma_post, sizeof(float) * hidden),
                                  rng(gamma_next, sizeof(float) * hidden)};
  if (boundary_alias(ins, rng(h, TH * 2), rng(h_out, TH * 2), rng(x_next, TH * 2), {}))
    return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  LAUNCH(7, beam::launch_boundary(b, nullptr, 0, nullptr, 0, 0, y, y_dtype == BEAM_BF16, T, hidden,
                                  st));
  return BEAM_OK;
}

beam_status_t beam_moe_forward_boundary(const void* x, const float* w_router, const float* bias,
                                        const void* w_gate_up, const void* w_down, int64_t T,
                                        const beam_moe_cfg* cfg, const float* w_gate_up_scale,
                                        const float* w_down_scale, const void* h,
                                        const float* gamma_post, const float* gamma_next,
                                        int32_t depth_n, float eps, void* h_out, void* x_next,
                                        int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  beam_status_t rc = check_cfg(cfg, true);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, true)) != BEAM_OK) return rc;
  const beam_moe_cfg& c = *cfg;
  if (c.x_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;   // the residual stream is bf16
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;
  if (!fp8 && (w_gate_up_scale || w_down_scale)) return BEAM_ERR_DTYPE;
  if (T == 0) return BEAM_OK;
  beam::BoundaryArgs bnd;
  if ((rc = make_boundary(h, gamma_post, gamma_next, h_out, x_next, c.hidden, depth_n, eps,
                          bnd)) != BEAM_OK)
    return rc;
  if (!x || !w_router || !bias || !w_gate_up || !w_down || !workspace) return BEAM_ERR_NULL;
  if (fp8 && (!w_gate_up_scale || !w_down_scale)) return BEAM_ERR_NULL;
  const void* ptrs[] = {x, w_router, bias, w_gate_up, w_down, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BEAM_ERR_ALIGN;
  if ((topk_ids_out && !aligned16(topk_ids_out)) || (topk_w_out && !aligned16(topk_w_out)) ||
      (w_gate_up_scale && !aligned16(w_gate_up_scale)) || (w_down_scale && !aligned16(w_down_scale)))
    return BEAM_ERR_ALIGN;
  const Layout L = make_layout(c, T, true);
  if (L.max_blocks > 65535) return BEAM_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;
  const size_t H = c.hidden, E = c.n_experts, F = c.d_ff, TK = (size_t)(T * c.topk);
  const size_t wb = dtype_bytes(c.w_dtype);
  std::vector<Range> ins = {rng(x, (size_t)T * H * 2), rng(w_router, sizeof(float) * E * H),
                            rng(bias, sizeof(float) * E), rng(w_gate_up, wb * E * 2 * F * H),
                            rng(w_down, wb * E * H * F), rng(gamma_post, sizeof(float) * H),
                            rng(gamma_next, sizeof(float) * H)};
  if (fp8) {
    ins.push_back(rng(w_gate_up_scale, sizeof(float) * E * 2 * F));
    ins.push_back(rng(w_down_scale, sizeof(float) * E * H));
  }
  std::vector<Range> outs = {rng(workspace, L.total)};
  if (topk_ids_out) outs.push_back(rng(topk_ids_out, sizeof(int32_t) * TK));
  if (topk_w_out) outs.push_back(rng(topk_w_out, sizeof(float) * TK));
  const size_t TH2 = (size_t)T * H * 2;
  if (boundary_alias(ins, rng(h, TH2), rng(h_out, TH2), rng(x_next, TH2), outs))
    return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* tw = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  const beam::Shape s = shape_of(c, T);
  if (beam::use_partial_route(s)) {
    float* part = reinterpret_cast<float*>(ws + L.sb);
    LAUNCH(0, beam::launch_router_partials(x, true, w_router, part, s, st));
    if (beam::use_fused_select_align(s)) {   // as in beam_moe_forward
      LAUNCH(1, beam::launch_select_align_small(part, bias, ids, tw, align_tables(L, ws), s, L.bm,
                                                st));
      return run_experts(c, T, L, ws, ids, tw, x, w_gate_up, w_down, w_gate_up_scale,
                         w_down_scale, nullptr, 0, c.n_experts, false, st, &bnd, 1, true);
    }
    LAUNCH(1, beam::launch_router_select_partials(part, bias, ids, tw, s, st));
  } else if ((rc = route_large(x, true, w_router, bias, ws + L.sb, ids, tw, s, st)) != BEAM_OK) {
    return rc;
  }
  return run_experts(c, T, L, ws, ids, tw, x, w_gate_up, w_down, w_gate_up_scale, w_down_scale,
                     nullptr, 0, c.n_experts, false, st, &bnd);
}

beam_status_t beam_moe_forward_routed(const void* x, const int32_t* topk_ids, const float* topk_w,
                                      const void* w_gate_up, const void* w_down, void* out,
                                      int64_t T, const beam_moe_cfg* cfg, int32_t expert_begin,
                                      int32_t expert_end, const float* w_gate_up_scale,
                                      const float* w_down_scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  beam_status_t rc = check_cfg(cfg, true);
  if (rc != BEAM_OK) return rc;
  if ((rc = check_T(cfg, T, true)) != BEAM_OK) return rc;
  const beam_moe_cfg& c = *cfg;
  if (expert_begin < 0 || expert_begin > expert_end || expert_end > c.n_experts)
    return BEAM_ERR_SHAPE;
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;
  if (!fp8 && (w_gate_up_scale || w_down_scale)) return BEAM_ERR_DTYPE;
  if (T == 0) return BEAM_OK;
  // an empty range has no local weights: those pointers may then be NULL
  const bool local = expert_begin < expert_end;
  if (!x || !topk_ids || !topk_w || !out || !workspace) return BEAM_ERR_NULL;
  if (local && (!w_gate_up || !w_down)) return BEAM_ERR_NULL;
  if (local && fp8 && (!w_gate_up_scale || !w_down_scale)) return BEAM_ERR_NULL;
  const void* ptrs[] = {x, topk_ids, topk_w, w_gate_up, w_down, out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return BEAM_ERR_ALIGN;
  if ((w_gate_up_scale && !aligned16(w_gate_up_scale)) ||
      (w_down_scale && !aligned16(w_down_scale)))
    return BEAM_ERR_ALIGN;
  const Layout L = make_layout(c, T, true);
  if (L.max_blocks > 65535) return BEAM_ERR_UNSUPPORTED;   // grid.y bound of the GEMM launches
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;

  const size_t H = c.hidden, F = c.d_ff, TK = (size_t)(T * c.topk);
  const size_t El = (size_t)(expert_end - expert_begin), wb = dtype_bytes(c.w_dtype);
  std::vector<Range> ins = {rng(x, (size_t)T * H * dtype_bytes(c.x_dtype)),
                            rng(topk_ids, sizeof(int32_t) * TK), rng(topk_w, sizeof(float) * TK),
                            rng(w_gate_up, wb * El * 2 * F * H), rng(w_down, wb * El * H * F)};
  if (fp8) {
    ins.push_back(rng(w_gate_up_scale, sizeof(float) * El * 2 * F));
    ins.push_back(rng(w_down_scale, sizeof(float) * El * H));
  }
  const std::vector<Range> outs = {rng(out, (size_t)T * H * dtype_bytes(c.out_dtype)),
                                   rng(workspace, L.total)};
  if (any_alias(ins, outs)) return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return run_experts(c, T, L, reinterpret_cast<char*>(workspace), topk_ids, topk_w, x, w_gate_up,
                     w_down, w_gate_up_scale, w_down_scale, out, expert_begin,
                     expert_end - expert_begin, true, st);
}

size_t beam_dense_mlp_workspace_bytes(int32_t hidden, int32_t d_ff, int32_t w_dtype, int64_t T) {
  if (check_dense(hidden, d_ff, w_dtype, BEAM_F32, T) != BEAM_OK) return 0;
  const beam_moe_cfg c = dense_cfg(hidden, d_ff, w_dtype, BEAM_F32);
  return make_layout(c, T, true, dense_ksplit_max(c, T)).total;
}

beam_status_t beam_dense_mlp_forward(const void* x, const void* w_gate_up, const void* w_down,
                                     void* out, int64_t T, int32_t hidden, int32_t d_ff,
                                     int32_t w_dtype, int32_t out_dtype,
                                     const float* w_gate_up_scale, const float* w_down_scale,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  beam_status_t rc = check_dense(hidden, d_ff, w_dtype, out_dtype, T);
  if (rc != BEAM_OK) return rc;
  const bool fp8 = w_dtype == BEAM_FP8_E4M3;
  if (!fp8 && (w_gate_up_scale || w_down_scale)) return BEAM_ERR_DTYPE;
  if (T == 0) return BEAM_OK;
  if (!x || !w_gate_up || !w_down || !out || !workspace) return BEAM_ERR_NULL;
  if (fp8 && (!w_gate_up_scale || !w_down_scale)) return BEAM_ERR_NULL;
  const void* ptrs[] = {x, w_gate_up, w_down, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BEAM_ERR_ALIGN;
  if ((w_gate_up_scale && !aligned16(w_gate_up_scale)) ||
      (w_down_scale && !aligned16(w_down_scale)))
    return BEAM_ERR_ALIGN;
  const beam_moe_cfg c = dense_cfg(hidden, d_ff, w_dtype, out_dtype);
  const int ks_max = dense_ksplit_max(c, T);
  const Layout L = make_layout(c, T, true, ks_max);
  if (L.max_blocks > 65535) return BEAM_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;
  const size_t H = hidden, F = d_ff, wb = dtype_bytes(w_dtype);
  std::vector<Range> ins = {rng(x, (size_t)T * H * 2), rng(w_gate_up, wb * 2 * F * H),
                            rng(w_down, wb * H * F)};
  if (fp8) {
    ins.push_back(rng(w_gate_up_scale, sizeof(float) * 2 * F));
    ins.push_back(rng(w_down_scale, sizeof(float) * H));
  }
  const std::vector<Range> outs = {rng(out, (size_t)T * H * dtype_bytes(out_dtype)),
                                   rng(workspace, L.total)};
  if (any_alias(ins, outs)) return BEAM_ERR_ALIAS;
  if ((rc = check_device()) != BEAM_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + L.ids);
  float* tw = reinterpret_cast<float*>(ws + L.w);
  if (launched(beam::launch_fill_dense_routes(ids, tw, T, st), st, "dense routes") != BEAM_OK)
    return BEAM_ERR_LAUNCH;
  // one expert: the tiled down GEMM has ceil(T / BM) x (hidden / 256) workgroups, few enough at
  // prefill sizes that a K split evens out the last round
  int ks = 1;
  if (ks_max > 1) {
    const int64_t tiles = ceil_div(T, (int64_t)L.bm) * (hidden / beam::kPipeDownCols);
    ks = std::min(ks_max, beam::down_ksplit(tiles, (int64_t)d_ff * dtype_bytes(w_dtype) / 128,
                                            device_cus()));
  }
  return run_experts(c, T, L, ws, ids, tw, x, w_gate_up, w_down, w_gate_up_scale, w_down_scale,
                     out, 0, 1, false, st, nullptr, ks);
}

beam_status_t beam_moe_quant_fp8(const void* src, int64_t rows, int32_t cols, uint8_t* codes,
                                 float* scales, void* stream) {
  if (rows < 0 || cols <= 0) return BEAM_ERR_SHAPE;
  if (cols % 8 != 0 || rows >= (int64_t(1) << 31)) return BEAM_ERR_UNSUPPORTED;
  if (rows == 0) return BEAM_OK;
  if (!src || !codes || !scales) return BEAM_ERR_NULL;
  if (!aligned16(src) || !aligned16(codes) || !aligned16(scales)) return BEAM_ERR_ALIGN;
  const size_t n = (size_t)rows * (size_t)cols;
  if (any_alias({rng(src, 2 * n)}, {rng(codes, n), rng(scales, sizeof(float) * (size_t)rows)}))
    return BEAM_ERR_ALIAS;
  beam_status_t rc = check_device();
  if (rc != BEAM_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return launched(beam::launch_quant_rows_fp8(reinterpret_cast<const uint16_t*>(src), rows, cols,
                                              codes, scales, st),
                  st, "quant_fp8");
}

beam_status_t beam_moe_convert(const float* src, int64_t n, int32_t dst_dtype, void* dst,
                               void* stream) {
  if (n < 0) return BEAM_ERR_SHAPE;
  if (dst_dtype != BEAM_BF16 && dst_dtype != BEAM_FP8_E4M3) return BEAM_ERR_DTYPE;
  if (n == 0) return BEAM_OK;
  if (!src || !dst) return BEAM_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return BEAM_ERR_ALIGN;
  const size_t nb = (size_t)n;
  if (any_alias({rng(src, 4 * nb)}, {rng(dst, nb * dtype_bytes(dst_dtype))})) return BEAM_ERR_ALIAS;
  beam_status_t rc = check_device();
  if (rc != BEAM_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return launched(beam::launch_convert(src, n, dst_dtype == BEAM_FP8_E4M3, dst, st), st,
                  "convert");
}

beam_status_t beam_moe_fp8_dot_tiles(const uint8_t* a, const uint8_t* b, const float* c, float* d,
                                     int64_t n_tiles, void* stream) {
  if (n_tiles < 0) return BEAM_ERR_SHAPE;
  if (n_tiles >= (int64_t(1) << 31)) return BEAM_ERR_UNSUPPORTED;
  if (n_tiles == 0) return BEAM_OK;
  if (!a || !b || !c || !d) return BEAM_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d)) return BEAM_ERR_ALIGN;
  const size_t n = (size_t)n_tiles;
  if (any_alias({rng(a, 2048 * n), rng(b, 2048 * n), rng(c, 1024 * n)}, {rng(d, 1024 * n)}))
    return BEAM_ERR_ALIAS;
  beam_status_t rc = check_device();
  if (rc != BEAM_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return launched(beam::launch_fp8_dot_tiles(a, b, c, d, n_tiles, st), st, "fp8_dot_tiles");
}

void beam_moe_timing_enable(int32_t enable) { g_timing = enable != 0; }

void beam_moe_timing_stages(uint32_t stage_mask) { g_timing_mask = stage_mask; }

int32_t beam_moe_timing_collect(double* total_ms, int32_t* launches, int32_t n_stages) {
  for (int i = 0; i < n_stages && i < kNumStages; ++i) {
    if (total_ms) total_ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (auto& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess &&
        r.stage < n_stages) {
      if (total_ms) total_ms[r.stage] += ms;
      if (launches) launches[r.stage] += 1;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
  return kNumStages;
}

const char* beam_moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : "unknown";
}

}  // extern "C"
