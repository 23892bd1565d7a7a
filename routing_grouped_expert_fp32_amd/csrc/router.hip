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
// router_select: one wave per token, no sort: group top-2 sums, group ranks by counting, then K
//   rounds of a wave-wide argmax (xor butterfly) over the kept groups' members; ties -> lower index.
#include "common.h"

namespace beam {

// ---------------------------------------------------------------------------------------------
// Logits. WG = 4 waves; WG tile = TM tokens x EB experts; wave w covers K range [w*H/4, (w+1)*H/4).
// Per 16-wide K step a lane loads 4 consecutive K values of one token row (A) and of one expert
// row (B); MFMA step c consumes component c, so step c sums K offsets {c, 4+c, 8+c, 12+c}: the same
// permutation on both operands, hence the same products.
template <bool XBF16, int TM, int EB>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float2* __restrict__ sb, int64_t T,
                                                            int H, int E) {
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
// Selection: one wave per token, 4 tokens per WG. Lane l owns experts l, l+64, l+128, l+192.
__device__ __forceinline__ bool better(float v1, int e1, float v2, int e2) {
  return v1 > v2 || (v1 == v2 && e1 < e2);
}

__global__ __launch_bounds__(256) void router_select_kernel(const float2* __restrict__ sb,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ wout, int64_t T,
                                                            int E, int G, int Gk, int K,
                                                            float scale) {
  __shared__ float bl[4][256];
  __shared__ float gsc[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave exits together; no block barrier below
  const int gs = E / G;
  float sv[4], bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      float2 p = sb[t * E + e];
      sv[j] = p.x;
      bv[j] = p.y;
      bl[wave][e] = p.y;
    } else {
      sv[j] = 0.f;
      bv[j] = -INFINITY;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  // group score: sum of the two largest b of the group (duplicates count twice)
  float myscore = -INFINITY;
  if (lane < G) {
    float v1 = -INFINITY, v2 = -INFINITY;
    for (int m = 0; m < gs; ++m) {
      const float v = bl[wave][lane * gs + m];
      if (v > v1) {
        v2 = v1;
        v1 = v;
      } else if (v > v2) {
        v2 = v;
      }
    }
    myscore = gs >= 2 ? v1 + v2 : v1;
    gsc[wave][lane] = myscore;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  bool kept_me = false;
  if (lane < G) {
    int rank = 0;
    for (int q = 0; q < G; ++q) {
      const float o = gsc[wave][q];
      rank += (o > myscore || (o == myscore && q < lane)) ? 1 : 0;
    }
    kept_me = rank < Gk;
  }
  const uint64_t kept = __ballot(kept_me);
  float cv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    cv[j] = (e < E && ((kept >> (e / gs)) & 1ull)) ? bv[j] : -INFINITY;
  }
  int my_id = 0;
  float my_s = 0.f, ssum = 0.f;
  for (int k = 0; k < K; ++k) {
    float v = cv[0];
    int e = lane;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (cv[j] > v) {  // strict: on equal values the lower expert (smaller j) stays
        v = cv[j];
        e = lane + 64 * j;
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off);
      const int oe = __shfl_xor(e, off);
      if (better(ov, oe, v, e)) {
        v = ov;
        e = oe;
      }
    }
    // every lane now holds the winner e; its owner retires it
    const int owner = e & 63, slotj = e >> 6;
    float s_win = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j == slotj) s_win = sv[j];
    s_win = __shfl(s_win, owner);
    if (lane == owner) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == slotj) cv[j] = -INFINITY;
    }
    ssum += s_win;
    if (lane == k) {
      my_id = e;
      my_s = s_win;
    }
  }
  if (lane < K) {
    ids[t * K + lane] = my_id;
    wout[t * K + lane] = scale * my_s / ssum;
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
    dim3 grid((unsigned)ceil_div(s.T, 32), s.E / 64);
    if (x_bf16)
      hipLaunchKernelGGL((router_logits_kernel<true, 32, 64>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
    else
      hipLaunchKernelGGL((router_logits_kernel<false, 32, 64>), grid, dim3(256), 0, st, x,
                         w_router, bias, sb, s.T, s.H, s.E);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const float2* sb, int32_t* ids, float* w, const Shape& s,
                                hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(s.T, 4));
  hipLaunchKernelGGL(router_select_kernel, grid, dim3(256), 0, st, sb, ids, w, s.T, s.E, s.G,
                     s.Gk, s.K, s.scale);
  return hipGetLastError();
}

}  // namespace beam
