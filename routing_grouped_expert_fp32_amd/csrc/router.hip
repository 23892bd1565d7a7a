// Router kernels of the Beam MoE block (gfx950).
//
// Sources: [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" §MoE and residual stream (FP32
// router weights, accumulation and logits; sigmoid scores plus correction bias pick 4 of 8 groups and
// then 8 experts; renormalised weights times 2.5), [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0
// 许可" §专家混合 (groups ranked by the sum of their two best scores), [S] "SGLang 原生支持 Reflection
// 的 Beam 并驱动其生产 API" §Dense Layers and Grouped MoE Routing (bias used to choose; FP32 routing
// coefficients).
//
// Three ways to the same logits (FP32 sums of exact products), chosen by batch size and dtype
// (host_rules.cpp):
// router_partial (up to 1024 tokens): logits = x . W_r^T on the FP32 matrix cores
//   (v_mfma_f32_16x16x4_f32), split over 256-wide hidden chunks into many workgroups (a few tokens
//   would leave W_r streamed by a few CUs); the selection sums the partial logits in chunk order.
// router_split + router_fused (bf16 x past 1024 tokens): W_r split exactly into three bf16 planes
//   once per call, then one workgroup per 32 tokens computes all 256 logits on the bf16 matrix
//   cores, keeps them in LDS and selects there: nothing but the routes leaves the chip.
// router_logits (FP32 x past 1024 tokens): FP32 matrix cores, 8 partial chains per output (4 waves
//   over K quarters, 2 alternating accumulators per wave) summed in a fixed order; writes
//   s = sigmoid(logit), b = s + bias[e] per (t, e) for router_select.
// router_select: one wave per token, no sort (route_select.h).
#include "device_common.h"
#include "route_select.h"

namespace beam {

// ---------------------------------------------------------------------------------------------
// Logits. WG = 4 waves; WG tile = TM tokens x EB experts; wave w covers K range [w*H/4, (w+1)*H/4).
// Per 16-wide K step a lane loads 4 consecutive K values of one token row (A) and of one expert
// row (B); MFMA step c consumes component c, so step c sums K offsets {c, 4+c, 8+c, 12+c}: the same
// permutation on both operands, hence the same products.
// Tiles past 64 tokens: 64 tokens x 64 experts (each workgroup reads its 1.3 MB W_r slice for twice
// as many tokens as with 32-token tiles: 0.275 -> 0.225 ms at T=8192 with bf16 x, 1.03 -> 0.845 ms
// at T=32768), two workgroups per CU by registers and LDS; 128-token tiles spill. Loading the next
// 16-deep step's operands ahead of the current MFMAs measured slower.
template <bool XBF16, int TM, int EB>
__global__ __launch_bounds__(256, TM >= 64 ? 2 : 4) void router_logits_kernel(
    const void* __restrict__ xv, const float* __restrict__ wr, const float* __restrict__ bias,
    float2* __restrict__ sb, int64_t T, int H, int E) {
  constexpr int MB = TM / 16, NB = EB / 16;
  __shared__ float part[4][TM][EB + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TM;
  const int e0 = blockIdx.y * EB;
  const int r = lane & 15, g = lane >> 4;
  const int kq = H / 4;
  const int kbeg = wave * kq;

  const float* bptr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) bptr[nb] = wr + (int64_t)(e0 + nb * 16 + r) * H + kbeg + 4 * g;
  int64_t arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int64_t t = t0 + mb * 16 + r;
    arow[mb] = (t < T ? t : T - 1) * H + kbeg + 4 * g;   // tail rows re-read a valid row
  }

  floatx4 acc[2][MB][NB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[c][mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < kq; k += 32) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kk = k + 16 * half;
      float a[MB][4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (XBF16) {
          const uint16_t* xp = reinterpret_cast<const uint16_t*>(xv) + arow[mb] + kk;
          u32x2 p = *reinterpret_cast<const u32x2*>(xp);
          a[mb][0] = bf16_lo(p.x); a[mb][1] = bf16_hi(p.x);
          a[mb][2] = bf16_lo(p.y); a[mb][3] = bf16_hi(p.y);
        } else {
          const float* xp = reinterpret_cast<const float*>(xv) + arow[mb] + kk;
          floatx4 p = *reinterpret_cast<const floatx4*>(xp);
          a[mb][0] = p.x; a[mb][1] = p.y; a[mb][2] = p.z; a[mb][3] = p.w;
        }
      }
      floatx4 b[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) b[nb] = *reinterpret_cast<const floatx4*>(bptr[nb] + kk);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[half][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb][c], b[nb][c],
                                                                      acc[half][mb][nb], 0, 0, 0);
    }
  }
  // D layout: lane holds rows 4g..4g+3 (tokens), column r (expert) of each 16x16 tile.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part[wave][mb * 16 + 4 * g + i][nb * 16 + r] = acc[0][mb][nb][i] + acc[1][mb][nb][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TM * EB; idx += 256) {
    const int tl = idx / EB, el = idx % EB;
    const int64_t t = t0 + tl;
    if (t >= T) continue;
    float z = ((part[0][tl][el] + part[1][tl][el]) + part[2][tl][el]) + part[3][tl][el];
    float s = 1.0f / (1.0f + expf(-z));
    float bsel = s + bias[e0 + el];
    sb[t * E + e0 + el] = make_float2(s, bsel);
  }
}

// ---------------------------------------------------------------------------------------------
// Logits for small batches (T <= kPartialRouteT): split over the hidden dimension so that enough
// workgroups stream W_r. WG (token tile of 16, expert tile of 16, hidden chunk of 256); wave w takes
// hidden [256 q + 64 w, 256 q + 64 w + 64), the four wave partials are summed in wave order and
// written to part[q][t][e]; the selection sums the chunks q in order.
template <bool XBF16>
__global__ __launch_bounds__(256) void router_partial_kernel(const void* __restrict__ xv,
                                                             const float* __restrict__ wr,
                                                             float* __restrict__ part, int64_t T,
                                                             int H, int E) {
  __shared__ float red[4][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int e0 = blockIdx.y * 16, q = blockIdx.z;
  const int r = lane & 15, g = lane >> 4;
  const int kbeg = q * 256 + wave * 64;
  const int64_t t = t0 + r;
  const int64_t arow = (t < T ? t : T - 1) * H + kbeg + 4 * g;   // tail rows re-read a valid row
  const float* bp = wr + (int64_t)(e0 + r) * H + kbeg + 4 * g;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 64; kk += 16) {
    float a[4];
    if constexpr (XBF16) {
      const u32x2 p = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(xv) + arow +
                                                      kk);
      a[0] = bf16_lo(p.x); a[1] = bf16_hi(p.x);
      a[2] = bf16_lo(p.y); a[3] = bf16_hi(p.y);
    } else {
      const floatx4 p = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(xv) +
                                                         arow + kk);
      a[0] = p.x; a[1] = p.y; a[2] = p.z; a[3] = p.w;
    }
    const floatx4 w4 = *reinterpret_cast<const floatx4*>(bp + kk);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], w4.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], w4.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], w4.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], w4.w, acc, 0, 0, 0);
  }
  // D layout: lane holds rows 4g..4g+3 (tokens), column r (expert)
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
  __syncthreads();
  const int tl = threadIdx.x >> 4, el = threadIdx.x & 15;
  if (t0 + tl < T) {
    const float z = ((red[0][tl][el] + red[1][tl][el]) + red[2][tl][el]) + red[3][tl][el];
    part[((int64_t)q * T + t0 + tl) * E + e0 + el] = z;
  }
}

// ---------------------------------------------------------------------------------------------
// One-pass router for bf16 activations (T > kPartialRouteT): logits, sigmoid, bias and selection in
// one workgroup per 32 tokens; the logits never leave the chip.
//
// Exact split of the FP32 weights, once per call (router_split_kernel): w = hi + mid + lo with three
// bf16 values (hi: w truncated to its leading 8 significant bits; mid: the leading 8 bits of the
// exact remainder w - hi; lo: the rest, at most 8 bits, so exact), valid for |w| >= 2^-102 (the
// remainders stay normal; smaller weights lose only bits below 2^-126, far below any logit's FP32
// rounding). A bf16 activation times each part is exact in FP32, so x.w = x.hi + x.mid + x.lo with
// no rounding before the FP32 accumulation of the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, 16x
// the FP32 MFMA rate: three products cost about a fifth of one FP32 MFMA pass). hi products go to
// one FP32 accumulator, mid and lo products to a second; z = acc_hi + acc_lo.
// The planes are stored in MFMA fragment order, so each wave load of the one-pass router reads
// 1 KB contiguous: fragment (expert tile nt, 32-deep step s, plane p) is 64 lanes x 8 bf16 at
// ((nt * H/32 + s) * 3 + p) * 512 elements, lane 16 g + r holding expert 16 nt + r, hidden
// 32 s + 8 g .. + 7.
constexpr int kSplitPerThread = 8;
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr,
                                                           uint16_t* __restrict__ planes,
                                                           int64_t n, int H) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kSplitPerThread;
  if (i >= n) return;   // n % 8 == 0 (H % 256 == 0)
  const int e = (int)(i / H), k0 = (int)(i % H);
  const int64_t frag = ((int64_t)(e >> 4) * (H / 32) + (k0 >> 5)) * 3;
  const int lane = 16 * ((k0 & 31) >> 3) + (e & 15);
  uint16_t* const dst = planes + frag * 512 + 8 * lane;
  const floatx4 a = *reinterpret_cast<const floatx4*>(wr + i);
  const floatx4 b = *reinterpret_cast<const floatx4*>(wr + i + 4);
  const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u32x4 h, m, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float v = w[2 * p + q];
      hb[q] = __float_as_uint(v) & 0xFFFF0000u;
      const float r1 = v - __uint_as_float(hb[q]);              // exact
      mb[q] = __float_as_uint(r1) & 0xFFFF0000u;
      lb[q] = __float_as_uint(r1 - __uint_as_float(mb[q]));     // exact, <= 8 significant bits
    }
    h[p] = (hb[0] >> 16) | hb[1];   // element 2p in the low half
    m[p] = (mb[0] >> 16) | mb[1];
    l[p] = (lb[0] >> 16) | (lb[1] & 0xFFFF0000u);
  }
  *reinterpret_cast<u32x4*>(dst) = h;
  *reinterpret_cast<u32x4*>(dst + 512) = m;
  *reinterpret_cast<u32x4*>(dst + 1024) = l;
}

// Scores of one token from its logits row in LDS.
struct ScoresFromLogits {
  const float* z;      // [E] logits of the token
  const float* bias;
  int E;
  __device__ void get4(int64_t, int lane, float* s, float* b) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E) {
        s[j] = 1.0f / (1.0f + expf(-z[e]));
        b[j] = s[j] + bias[e];
      }
    }
  }
};

// WG = 8 waves, kRfTM tokens (32; 64 past 8192 tokens) x all E experts (E <= 256, E % 16 == 0).
// Wave w owns the expert tiles w and w + 8 (16 experts each) for every 16-token tile, over the
// whole hidden dimension, in 32-deep MFMA steps. Token rows go through an LDS ring of 256-wide
// hidden chunks (rows padded to 528 B so the 16 rows of a fragment read fall on distinct banks),
// loaded into registers one chunk ahead and stored after the chunk's MFMAs; each wave's weight
// fragments (three planes) stream from L2 straight into registers, kPrefW steps ahead. Then the
// logits go to LDS and each wave selects kRfTM / 8 tokens (select_token).
// Past 8192 tokens the workgroups take 64 tokens (half the weight stream per token; a workgroup's
// time is set by its 7.5 MB weight stream either way), with two weight steps in flight.
constexpr int kRfWaves = 8, kRfChunk = 256, kRfRowBytes = 2 * kRfChunk + 16;
constexpr int kRfSteps = kRfChunk / 32;   // MFMA steps per chunk
constexpr int64_t kRfWideT = 8192;        // batches past this use 64-token workgroups
template <int kRfTM, int kPrefW>
__global__ __launch_bounds__(64 * kRfWaves, 1) void router_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ wout, int64_t T,
    int H, int E, int G, int Gk, int K, float scale) {
  constexpr int MB = kRfTM / 16, NB = 2;
  // token-row chunk: kRfTM rows x 32 16-byte pieces, TPR threads per row, PPT pieces each
  constexpr int TPR = 64 * kRfWaves / kRfTM, PPT = 32 / TPR;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][kRfTM * kRfRowBytes];
  __shared__ float zl[kRfTM][256 + 1];
  __shared__ float bl[kRfWaves][256];
  __shared__ float gsc[kRfWaves][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kRfTM;
  const int n_et = E / 16;

  // token-row chunk loads: thread -> row tid / TPR, 16-byte pieces tid % TPR + TPR i, i < PPT
  const int xr = tid / TPR, xc = tid % TPR;
  const int64_t xrow = min(t0 + xr, T - 1);   // tail rows re-read a valid row
  const uint16_t* xsrc = x + xrow * H + 8 * xc;
  u32x4 xv[PPT];
  auto load_x = [&](int chunk) {
    const uint16_t* p = xsrc + chunk * kRfChunk;
#pragma unroll
    for (int i = 0; i < PPT; ++i) xv[i] = *reinterpret_cast<const u32x4*>(p + 8 * TPR * i);
  };
  auto store_x = [&](int slot) {
    unsigned char* d = xs[slot] + xr * kRfRowBytes + 16 * xc;
#pragma unroll
    for (int i = 0; i < PPT; ++i) *reinterpret_cast<u32x4*>(d + 16 * TPR * i) = xv[i];
  };

  // weight fragments of expert tile nt = wave + 8 i, in fragment order (router_split_kernel): lane
  // 16 g + r gets expert 16 nt + r, hidden 8 g .. 8 g + 7 of each step and plane (tiles past E
  // read tile 0 and are discarded)
  const int nsteps = H / 32;
  const uint16_t* wsrc[NB];
  bool wvalid[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int nt = wave + kRfWaves * i;
    wvalid[i] = nt < n_et;
    wsrc[i] = planes + (int64_t)(wvalid[i] ? nt : 0) * nsteps * 3 * 512 + 8 * lane;
  }
  bf16x8 wb[kPrefW][NB][3];
  auto load_w = [&](int buf, int step) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int p = 0; p < 3; ++p)
        wb[buf][i][p] = *reinterpret_cast<const bf16x8*>(wsrc[i] + (3 * step + p) * 512);
  };

  floatx4 acc_h[MB][NB], acc_l[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      acc_h[m][i] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc_l[m][i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  load_x(0);
  store_x(0);
  // the prologue issues the ring in the steady-state order (oldest first), so the first wait of
  // the loop is as partial as the others
#pragma unroll
  for (int u = 0; u < kPrefW; ++u) {
    load_w(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nchunks = H / kRfChunk;
  static_assert(kRfSteps % kPrefW == 0, "weight ring turns over within a chunk");
  // Loads and MFMAs are unconditional inside the loop (past the end they re-read the last chunk /
  // step, and tiles past E compute on tile 0's rows and are discarded), so the loop has no branches
  // and the weight ring stays in fixed registers with partial vmcnt waits.
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();   // chunk c is in LDS; everyone is done with chunk c - 1's slot
    load_x(min(c + 1, nchunks - 1));
    const unsigned char* sa = xs[c & 1];
#pragma unroll
    for (int s0 = 0; s0 < kRfSteps; s0 += kPrefW) {
#pragma unroll
      for (int u = 0; u < kPrefW; ++u) {
        const int step = c * kRfSteps + s0 + u;
        bf16x8 af[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
          af[m] = *reinterpret_cast<const bf16x8*>(sa + (16 * m + r) * kRfRowBytes +
                                                   64 * (s0 + u) + 16 * g);
        bf16x8 bw[NB][3];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int p = 0; p < 3; ++p) bw[i][p] = wb[u][i][p];
        load_w(u, min(step + kPrefW, nsteps - 1));
        // keep the prefetch here: without this fence the scheduler sinks each load next to its
        // use four steps later and waits for it there
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            acc_h[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bw[i][0], acc_h[m][i], 0,
                                                                  0, 0);
            acc_l[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bw[i][1], acc_l[m][i], 0,
                                                                  0, 0);
            acc_l[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bw[i][2], acc_l[m][i], 0,
                                                                  0, 0);
          }
      }
    }
    store_x((c + 1) & 1);   // (the last chunk stores into the idle slot)
  }
  // logits to LDS: lane holds tokens 4 g + q, expert 16 nt + r of each tile
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (!wvalid[i]) continue;
    const int e = 16 * (wave + kRfWaves * i) + r;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) zl[16 * m + 4 * g + q][e] = acc_h[m][i][q] + acc_l[m][i][q];
  }
  __syncthreads();
  for (int tl = wave; tl < kRfTM; tl += kRfWaves) {
    const int64_t t = t0 + tl;
    if (t >= T) break;   // wave-uniform
    int id;
    float w;
    select_token(ScoresFromLogits{zl[tl], bias, E}, t, lane, bl[wave], gsc[wave], E, G, Gk, K,
                 scale, id, w);
    if (lane < K) {
      ids[t * K + lane] = id;
      wout[t * K + lane] = w;
    }
  }
}

static_assert(kRfChunk == kRouterChunk && kMaxChunks == kRouterMaxChunks, "router chunking");

hipError_t launch_router_split(const float* w_router, uint16_t* planes, const Shape& s,
                               hipStream_t st) {
  const int64_t n = (int64_t)s.E * s.H;
  if (n % kSplitPerThread) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)ceil_div(n / kSplitPerThread, 256)),
                     dim3(256), 0, st, w_router, planes, n, s.H);
  return hipGetLastError();
}

hipError_t launch_router_fused(const void* x, const uint16_t* planes, const float* bias,
                               int32_t* ids, float* w, const Shape& s, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (!use_fused_router(s, true)) return hipErrorInvalidValue;
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  if (s.T > kRfWideT)
    hipLaunchKernelGGL((router_fused_kernel<64, 2>), dim3((unsigned)ceil_div(s.T, 64)),
                       dim3(64 * kRfWaves), 0, st, xb, planes, bias, ids, w, s.T, s.H, s.E, s.G,
                       s.Gk, s.K, s.scale);
  else
    hipLaunchKernelGGL((router_fused_kernel<32, 4>), dim3((unsigned)ceil_div(s.T, 32)),
                       dim3(64 * kRfWaves), 0, st, xb, planes, bias, ids, w, s.T, s.H, s.E, s.G,
                       s.Gk, s.K, s.scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Selection: one wave per token, 4 tokens per WG (select_token in route_select.h).
template <class Src>
__global__ __launch_bounds__(256) void router_select_kernel(Src src, int32_t* __restrict__ ids,
                                                            float* __restrict__ wout, int64_t T,
                                                            int E, int G, int Gk, int K,
                                                            float scale) {
  __shared__ float bl[4][256];
  __shared__ float gsc[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave exits together; no block barrier below
  int id;
  float w;
  select_token(src, t, lane, bl[wave], gsc[wave], E, G, Gk, K, scale, id, w);
  if (lane < K) {
    ids[t * K + lane] = id;
    wout[t * K + lane] = w;
  }
}

hipError_t launch_router_logits(const void* x, bool x_bf16, const float* w_router,
                                const float* bias, float2* sb, const Shape& s, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.T <= 64 || s.E < 64) {
    dim3 grid((unsigned)ceil_div(s.T, 16), s.E / 16);
    if (x_bf16)
      hipLaunchKernelGGL((router_logits_kernel<true, 16, 16>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
    else
      hipLaunchKernelGGL((router_logits_kernel<false, 16, 16>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
  } else {
    dim3 grid((unsigned)ceil_div(s.T, 64), s.E / 64);
    if (x_bf16)
      hipLaunchKernelGGL((router_logits_kernel<true, 64, 64>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
    else
      hipLaunchKernelGGL((router_logits_kernel<false, 64, 64>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const float2* sb, int32_t* ids, float* w, const Shape& s,
                                hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 4));
  hipLaunchKernelGGL(router_select_kernel<ScoresFromPairs>, grid, dim3(256), 0, st,
                     ScoresFromPairs{sb, s.E}, ids, w, s.T, s.E, s.G, s.Gk, s.K, s.scale);
  return hipGetLastError();
}

hipError_t launch_router_select_partials(const float* part, const float* bias, int32_t* ids,
                                         float* w, const Shape& s, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 4));
  const ScoresFromPartials src{part, bias, router_partial_chunks(s), s.T, s.E};
  hipLaunchKernelGGL(router_select_kernel<ScoresFromPartials>, grid, dim3(256), 0, st, src, ids, w,
                     s.T, s.E, s.G, s.Gk, s.K, s.scale);
  return hipGetLastError();
}

hipError_t launch_router_partials(const void* x, bool x_bf16, const float* w_router, float* part,
                                  const Shape& s, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 16), s.E / 16, router_partial_chunks(s));
  if (x_bf16)
    hipLaunchKernelGGL(router_partial_kernel<true>, grid, dim3(256), 0, st, x, w_router, part,
                       s.T, s.H, s.E);
  else
    hipLaunchKernelGGL(router_partial_kernel<false>, grid, dim3(256), 0, st, x, w_router, part,
                       s.T, s.H, s.E);
  return hipGetLastError();
}


}  // namespace beam
