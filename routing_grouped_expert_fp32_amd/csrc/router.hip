// Router kernels of the Beam MoE block (gfx950).
//
// Sources: [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" §MoE and residual stream (FP32
// router weights, accumulation and logits; sigmoid scores plus correction bias pick 4 of 8 groups and
// then 8 experts; renormalised weights times 2.5), [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0
// 许可" §专家混合 (groups ranked by the sum of their two best scores), [S] "SGLang 原生支持 Reflection
// 的 Beam 并驱动其生产 API" §Dense Layers and Grouped MoE Routing (bias used to choose; FP32 routing
// coefficients).
//
// router_logits: logits = x . W_r^T on the FP32 matrix cores (v_mfma_f32_16x16x4_f32). Accuracy:
//   the 5120-long dot products are split into 8 partial chains per output (4 waves over K quarters,
//   2 alternating accumulators per wave), summed in a fixed order, so the FP32 rounding error stays
//   ~8x below a single serial chain. Output per (t, e): s = sigmoid(logit), b = s + bias[e].
// router_partial (small batches): the same products split over 256-wide hidden chunks into more
//   workgroups (a handful of tokens would leave W_r streamed by a few CUs); partial logits are
//   summed in chunk order by the selection.
// router_select: one wave per token, no sort (route_select.h).
#include "common.h"
#include "route_select.h"

namespace beam {

// ---------------------------------------------------------------------------------------------
// Logits. WG = 4 waves; WG tile = TM tokens x EB experts; wave w covers K range [w*H/4, (w+1)*H/4).
// Per 16-wide K step a lane loads 4 consecutive K values of one token row (A) and of one expert
// row (B); MFMA step c consumes component c, so step c sums K offsets {c, 4+c, 8+c, 12+c}: the same
// permutation on both operands, hence the same products.
// Tiles for T > 64: 64 tokens x 64 experts (each workgroup reads its 1.3 MB W_r slice for twice
// as many tokens as with 32-token tiles: 0.275 -> 0.225 ms at T=8192, 1.03 -> 0.845 ms at
// T=32768), two workgroups per CU by registers and LDS; 128-token tiles spill. Loading the next
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
// Logits for small batches (T <= kSmallRouteT): split over the hidden dimension so that enough
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

int router_partial_chunks(const Shape& s) { return s.H / 256; }

bool use_small_route(const Shape& s) {
  return s.T <= kSmallRouteT && router_partial_chunks(s) <= kMaxChunks;
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
