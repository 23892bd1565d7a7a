// Sanitizer driver for the host side of the library (tests/test_abi.py builds it with
// -fsanitize=address,undefined and runs it on the CPU): every entry point over a range of shapes,
// batch sizes and dtypes, with each launch's buffers checked against the ones passed in (stubs.cpp),
// plus the validation errors. "Device" buffers are reserved address ranges that nothing reads.
#include <sys/mman.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/beam_moe.h"
#include "hostcheck.h"

namespace {

int g_calls = 0, g_fail = 0;

void expect(bool ok, const char* what, long a = 0, long b = 0) {
  ++g_calls;
  if (!ok) {
    ++g_fail;
    std::fprintf(stderr, "FAIL: %s (%ld, %ld)\n", what, a, b);
  }
}

// A reserved, never-touched address range of `bytes` (page-aligned), registered for the stubs.
void* dev(size_t bytes, const char* name) {
  const size_t n = bytes ? (bytes + 4095) & ~size_t(4095) : 4096;
  void* p = mmap(nullptr, n, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
  if (p == MAP_FAILED) {
    std::perror("mmap");
    std::exit(2);
  }
  hostcheck::register_range(p, bytes, name);
  return p;
}

std::vector<std::pair<void*, size_t>> g_maps;
void* buf(size_t bytes, const char* name) {
  void* p = dev(bytes, name);
  g_maps.push_back({p, bytes ? (bytes + 4095) & ~size_t(4095) : 4096});
  return p;
}
void release() {
  for (auto& m : g_maps) munmap(m.first, m.second);
  g_maps.clear();
  hostcheck::clear_ranges();
  hostcheck::register_range(hostcheck::scratch_range(), size_t(64) << 20, "scratch");
}

size_t dtb(int32_t dt) { return dt == BEAM_F32 ? 4 : dt == BEAM_BF16 ? 2 : 1; }

beam_moe_cfg cfg_of(int H, int E, int G, int Gk, int K, int F, int xd, int wd, int od) {
  beam_moe_cfg c;
  c.hidden = H;
  c.n_experts = E;
  c.n_groups = G;
  c.topk_groups = Gk;
  c.topk = K;
  c.d_ff = F;
  c.routed_scale = 2.5f;
  c.x_dtype = xd;
  c.w_dtype = wd;
  c.out_dtype = od;
  return c;
}

// All entry points of one cfg and batch size on valid arguments.
void valid_calls(const beam_moe_cfg& c, int64_t T) {
  const size_t H = c.hidden, E = c.n_experts, F = c.d_ff, K = c.topk;
  const bool fp8 = c.w_dtype == BEAM_FP8_E4M3;
  void* x = buf(T * H * dtb(c.x_dtype), "x");
  float* wr = (float*)buf(4 * E * H, "w_router");
  float* bias = (float*)buf(4 * E, "bias");
  void* wgu = buf(E * 2 * F * H * dtb(c.w_dtype), "w_gate_up");
  void* wdn = buf(E * H * F * dtb(c.w_dtype), "w_down");
  float* sgu = fp8 ? (float*)buf(4 * E * 2 * F, "w_gate_up_scale") : nullptr;
  float* sdn = fp8 ? (float*)buf(4 * E * H, "w_down_scale") : nullptr;
  void* out = buf(T * H * dtb(c.out_dtype), "out");
  int32_t* ids = (int32_t*)buf(4 * T * K, "topk_ids");
  float* tw = (float*)buf(4 * T * K, "topk_w");
  const long l0 = hostcheck::launches();

  const size_t rws = beam_moe_route_workspace_bytes(&c, T);
  void* rw = buf(rws, "route workspace");
  int rc = beam_moe_route(x, wr, bias, ids, tw, T, &c, rw, rws, nullptr);
  expect(rc == BEAM_OK, "route", rc, T);

  const size_t wsb = beam_moe_workspace_bytes(&c, T);
  expect(wsb > 0, "workspace bytes", T);
  void* ws = buf(wsb, "workspace");
  rc = beam_moe_forward(x, wr, bias, wgu, wdn, out, T, &c, sgu, sdn, ids, tw, ws, wsb, nullptr);
  expect(rc == BEAM_OK, "forward", rc, T);
  rc = beam_moe_forward(x, wr, bias, wgu, wdn, out, T, &c, sgu, sdn, nullptr, nullptr, ws, wsb,
                        nullptr);
  expect(rc == BEAM_OK, "forward without route copies", rc, T);
  rc = beam_moe_forward_noalloc(x, wr, bias, wgu, wdn, out, T, &c, sgu, sdn, ids, tw, nullptr);
  expect(rc == (wsb <= (size_t(64) << 20) ? BEAM_OK : BEAM_ERR_WORKSPACE), "noalloc", rc, T);

  const int32_t ranges[][2] = {{0, (int32_t)E}, {(int32_t)E / 4, (int32_t)E / 2},
                               {(int32_t)E / 2, (int32_t)E / 2}, {(int32_t)E - 1, (int32_t)E}};
  for (auto& r : ranges) {
    const size_t El = r[1] - r[0];
    const size_t wb = dtb(c.w_dtype);
    // local weights: a sub-range of the full arrays
    const void* lgu = El ? (const char*)wgu + r[0] * 2 * F * H * wb : nullptr;
    const void* ldn = El ? (const char*)wdn + r[0] * H * F * wb : nullptr;
    const float* lsgu = fp8 && El ? sgu + r[0] * 2 * F : nullptr;
    const float* lsdn = fp8 && El ? sdn + r[0] * H : nullptr;
    rc = beam_moe_forward_routed(x, ids, tw, lgu, ldn, out, T, &c, r[0], r[1], lsgu, lsdn, ws, wsb,
                                 nullptr);
    expect(rc == BEAM_OK, "routed", rc, r[0]);
  }

  for (int32_t region = 0; region <= 7; ++region) {
    size_t off = 0, bytes = 0;
    rc = beam_moe_workspace_region(&c, T, region, &off, &bytes);
    const bool fp8_only = region >= 3 && region <= 6;
    if (fp8_only && !fp8) {
      expect(rc == BEAM_ERR_UNSUPPORTED, "region unsupported", region, rc);
    } else {
      expect(rc == BEAM_OK && off % 256 == 0 && off + bytes <= wsb, "region inside workspace",
             region, (long)(off + bytes) - (long)wsb);
    }
  }

  if (c.x_dtype == BEAM_BF16 && c.hidden <= 16384) {
    void* h = buf(2 * T * H, "h");
    float* gp = (float*)buf(4 * H, "gamma_post");
    float* gn = (float*)buf(4 * H, "gamma_next");
    void* xn = buf(2 * T * H, "x_next");
    rc = beam_moe_forward_boundary(x, wr, bias, wgu, wdn, T, &c, sgu, sdn, h, gp, gn, 61, 1e-6f,
                                   h, xn, ids, tw, ws, wsb, nullptr);
    expect(rc == BEAM_OK, "forward_boundary (in place)", rc, T);
    rc = beam_residual_boundary(out, c.out_dtype, h, gp, gn, h, xn, T, c.hidden, 61, 1e-6f,
                                nullptr);
    expect(rc == BEAM_OK, "residual_boundary", rc, T);
  }
  if (T > 0) expect(hostcheck::launches() > l0, "launches reached the stubs", T);
  release();
}

void dense_calls(int H, int F, int32_t wd, int32_t od, int64_t T) {
  const bool fp8 = wd == BEAM_FP8_E4M3;
  void* x = buf(2 * T * H, "x");
  void* wgu = buf((size_t)2 * F * H * dtb(wd), "w_gate_up");
  void* wdn = buf((size_t)H * F * dtb(wd), "w_down");
  float* sgu = fp8 ? (float*)buf(8 * (size_t)F, "w_gate_up_scale") : nullptr;
  float* sdn = fp8 ? (float*)buf(4 * (size_t)H, "w_down_scale") : nullptr;
  void* out = buf(T * H * dtb(od), "out");
  const size_t wsb = beam_dense_mlp_workspace_bytes(H, F, wd, T);
  void* ws = buf(wsb, "dense workspace");
  int rc = beam_dense_mlp_forward(x, wgu, wdn, out, T, H, F, wd, od, sgu, sdn, ws, wsb, nullptr);
  expect(rc == BEAM_OK, "dense", rc, T);
  for (int32_t region = 0; region <= 7; ++region) {
    size_t off = 0, bytes = 0;
    rc = beam_dense_mlp_workspace_region(H, F, wd, T, region, &off, &bytes);
    if (rc == BEAM_OK) expect(off + bytes <= wsb, "dense region inside workspace", region, T);
  }
  release();
}

// Validation failures: each returns its status and reaches no launcher.
void invalid_calls() {
  beam_moe_cfg c = cfg_of(512, 32, 8, 2, 4, 256, BEAM_BF16, BEAM_BF16, BEAM_F32);
  const int64_t T = 40;
  void* x = buf(2 * T * 512, "x");
  float* wr = (float*)buf(4 * 32 * 512, "w_router");
  float* bias = (float*)buf(4 * 32, "bias");
  void* wgu = buf(32 * 512 * 512 * 2, "w_gate_up");
  void* wdn = buf(32 * 512 * 256 * 2, "w_down");
  void* out = buf(4 * T * 512, "out");
  const size_t wsb = beam_moe_workspace_bytes(&c, T);
  void* ws = buf(wsb, "workspace");
  float* sc = (float*)buf(4096, "scales");
  const long l0 = hostcheck::launches();
  auto fwd = [&](const beam_moe_cfg* cp, int64_t t, const void* xx, void* oo, void* w, size_t wb,
                 const float* s1, const float* s2) {
    return beam_moe_forward(xx, wr, bias, wgu, wdn, oo, t, cp, s1, s2, nullptr, nullptr, w, wb,
                            nullptr);
  };
  expect(fwd(nullptr, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_NULL, "null cfg");
  expect(fwd(&c, -1, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_SHAPE, "T < 0");
  expect(fwd(&c, T, nullptr, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_NULL, "null x");
  expect(fwd(&c, T, (char*)x + 2, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_ALIGN, "misaligned");
  expect(fwd(&c, T, x, out, ws, wsb - 1, nullptr, nullptr) == BEAM_ERR_WORKSPACE, "small ws");
  expect(fwd(&c, T, x, x, ws, wsb, nullptr, nullptr) == BEAM_ERR_ALIAS, "out aliases x");
  expect(fwd(&c, T, x, out, ws, wsb, sc, sc) == BEAM_ERR_DTYPE, "scales with bf16 experts");
  beam_moe_cfg b = c;
  b.n_groups = 7;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_SHAPE, "E % G != 0");
  b = c;
  b.topk = 20;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_SHAPE, "K > Gk E / G");
  b = c;
  b.hidden = 500;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_UNSUPPORTED, "H % 256");
  b = c;
  b.x_dtype = BEAM_F32;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_DTYPE, "f32 x, bf16 experts");
  b = c;
  b.w_dtype = 7;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_DTYPE, "unknown dtype");
  b = c;
  b.routed_scale = NAN;
  expect(fwd(&b, T, x, out, ws, wsb, nullptr, nullptr) == BEAM_ERR_SHAPE, "NaN routed_scale");
  b = c;
  b.w_dtype = BEAM_FP8_E4M3;
  const size_t wsb8 = beam_moe_workspace_bytes(&b, T);
  void* ws8 = buf(wsb8, "fp8 workspace");
  expect(fwd(&b, T, x, out, ws8, wsb8, nullptr, sc) == BEAM_ERR_NULL, "FP8 without scales");
  int32_t* ids = (int32_t*)buf(4 * T * 4, "ids");
  float* tw = (float*)buf(4 * T * 4, "w");
  expect(beam_moe_forward_routed(x, ids, tw, wgu, wdn, out, T, &c, 5, 3, nullptr, nullptr, ws,
                                 wsb, nullptr) == BEAM_ERR_SHAPE,
         "routed begin > end");
  expect(beam_moe_forward_routed(x, ids, tw, wgu, wdn, out, T, &c, 0, 33, nullptr, nullptr, ws,
                                 wsb, nullptr) == BEAM_ERR_SHAPE,
         "routed end > E");
  expect(beam_moe_route(x, wr, bias, ids, tw, T, &c, ws, 16, nullptr) == BEAM_ERR_WORKSPACE,
         "route small workspace");
  expect(beam_moe_route(x, wr, bias, (int32_t*)x, tw, T, &c, ws, wsb, nullptr) == BEAM_ERR_ALIAS,
         "route ids alias x");
  float* g = (float*)buf(4 * 512, "gamma");
  void* h = buf(2 * T * 512, "h");
  void* xn = buf(2 * T * 512, "x_next");
  expect(beam_residual_boundary(out, BEAM_F32, h, g, g, h, xn, T, 512, 0, 1e-6f, nullptr) ==
             BEAM_ERR_SHAPE,
         "boundary depth 0");
  expect(beam_residual_boundary(out, BEAM_F32, h, g, g, h, xn, T, 512, 4, NAN, nullptr) ==
             BEAM_ERR_SHAPE,
         "boundary NaN eps");
  expect(beam_residual_boundary(out, BEAM_F32, h, g, g, h, h, T, 512, 4, 1e-6f, nullptr) ==
             BEAM_ERR_ALIAS,
         "boundary x_next aliases h");
  expect(beam_dense_mlp_forward(x, wgu, wdn, out, T, 512, 256, BEAM_F32, BEAM_F32, nullptr,
                                nullptr, ws, wsb, nullptr) != BEAM_OK,
         "dense f32 weights");
  expect(beam_moe_convert(sc, 16, 9, out, nullptr) == BEAM_ERR_DTYPE, "convert dtype");
  expect(beam_moe_convert(sc, -1, BEAM_BF16, out, nullptr) == BEAM_ERR_SHAPE, "convert n < 0");
  size_t off, bytes;
  expect(beam_moe_workspace_region(&c, T, 99, &off, &bytes) != BEAM_OK, "unknown region");
  expect(beam_moe_workspace_region(&c, T, 0, nullptr, &bytes) == BEAM_ERR_NULL, "region null");
  expect(beam_moe_workspace_bytes(&b, -5) == 0, "workspace bytes of T < 0");
  expect(hostcheck::launches() == l0, "no launch on a validation failure",
         hostcheck::launches() - l0);
  release();
}

void misc_calls() {
  const int64_t n = 1000;
  float* src = (float*)buf(4 * n, "src");
  void* dst = buf(2 * n, "dst");
  expect(beam_moe_convert(src, n, BEAM_BF16, dst, nullptr) == BEAM_OK, "convert bf16");
  expect(beam_moe_convert(src, n, BEAM_FP8_E4M3, dst, nullptr) == BEAM_OK, "convert fp8");
  uint8_t* a = (uint8_t*)buf(2048 * 3, "a");
  uint8_t* bb = (uint8_t*)buf(2048 * 3, "b");
  float* c = (float*)buf(1024 * 3, "c");
  float* d = (float*)buf(1024 * 3, "d");
  expect(beam_moe_fp8_dot_tiles(a, bb, c, d, 3, nullptr) == BEAM_OK, "fp8 dot tiles");
  void* q = buf(2 * 77 * 512, "quant src");
  uint8_t* codes = (uint8_t*)buf(77 * 512, "codes");
  float* scales = (float*)buf(4 * 77, "scales");
  expect(beam_moe_quant_fp8(q, 77, 512, codes, scales, nullptr) == BEAM_OK, "quant fp8");
  for (int s = -1; s <= 12; ++s) expect(beam_status_string(s) != nullptr, "status string", s);
  expect(beam_moe_version() > 0, "version");
  // stage timing over one forward
  beam_moe_timing_enable(1);
  beam_moe_timing_stages(~0u);
  beam_moe_cfg cf = cfg_of(512, 32, 8, 2, 4, 256, BEAM_BF16, BEAM_BF16, BEAM_F32);
  release();
  valid_calls(cf, 100);
  double ms[8];
  int32_t cnt[8];
  const int32_t ns = beam_moe_timing_collect(ms, cnt, 8);
  expect(ns == 8, "stage count", ns);
  for (int i = 0; i < 8; ++i) expect(beam_moe_stage_name(i) != nullptr, "stage name", i);
  beam_moe_timing_enable(0);
  release();
}

}  // namespace

void* hostcheck::scratch_range() {
  static void* p = mmap(nullptr, size_t(64) << 20, PROT_NONE,
                        MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
  return p;
}

int main(int argc, char** argv) {
  const bool sync = argc > 1 && std::strcmp(argv[1], "--sync") == 0;
  if (sync) setenv("BEAM_MOE_SYNC_CHECK", "1", 1);
  release();
  const int64_t Ts[] = {0, 1, 3, 16, 17, 64, 65, 100, 321, 1000, 4096, 8192, 32768};
  std::vector<beam_moe_cfg> cfgs = {
      cfg_of(5120, 256, 8, 4, 8, 2560, BEAM_BF16, BEAM_BF16, BEAM_F32),
      cfg_of(5120, 256, 8, 4, 8, 2560, BEAM_BF16, BEAM_BF16, BEAM_BF16),
      cfg_of(5120, 256, 8, 4, 8, 2560, BEAM_BF16, BEAM_FP8_E4M3, BEAM_F32),
      cfg_of(512, 32, 8, 2, 4, 256, BEAM_F32, BEAM_F32, BEAM_F32),
      cfg_of(1024, 64, 8, 4, 6, 512, BEAM_BF16, BEAM_BF16, BEAM_F32),
      cfg_of(512, 128, 4, 2, 8, 256, BEAM_BF16, BEAM_FP8_E4M3, BEAM_BF16),
      cfg_of(768, 48, 3, 2, 5, 512, BEAM_BF16, BEAM_BF16, BEAM_F32),
  };
  for (const auto& c : cfgs)
    for (int64_t T : Ts) valid_calls(c, T);
  for (int64_t T : {int64_t(1), int64_t(32), int64_t(700), int64_t(8192)}) {
    dense_calls(5120, 20480, BEAM_BF16, BEAM_F32, T);
    dense_calls(5120, 20480, BEAM_FP8_E4M3, BEAM_BF16, T);
    dense_calls(512, 1024, BEAM_BF16, BEAM_F32, T);
  }
  invalid_calls();
  misc_calls();
  // BEAM_MOE_SYNC_CHECK: one synchronisation after every launch, none otherwise
  expect(hostcheck::syncs() == (sync ? hostcheck::launches() : 0), "synchronisations",
         hostcheck::syncs(), hostcheck::launches());
  std::printf("hostcheck: %d checks, %d failed, %ld launches checked\n", g_calls, g_fail,
              hostcheck::launches());
  return g_fail ? 1 : 0;
}
