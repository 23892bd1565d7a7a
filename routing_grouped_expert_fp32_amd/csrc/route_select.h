// Group-limited top-k selection of one token by one wave (gfx950), shared by the selection kernels.
//
// Sources: [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" §MoE and residual stream (sigmoid
// scores plus correction bias pick 4 of 8 groups, then 8 experts; renormalised weights times 2.5),
// [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" §专家混合 (groups ranked by the sum of their
// two best scores), [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" §Dense Layers and
// Grouped MoE Routing (the bias is used to choose only).
//
// No sort: lane l owns experts l, l+64, l+128, l+192; group top-2 sums by the group's first lanes,
// group ranks by counting, then K rounds of a wave-wide argmax (DPP row steps and four lane reads)
// over the kept groups' members. Ties go to the lower group / expert index.
#pragma once
#include "device_common.h"

namespace beam {

// Wave-wide max / min of a 32-bit unsigned value, returned to every lane: DPP steps inside each row
// of 16 lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row results read as
// scalars.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t rows_u32(uint32_t v, int i) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * i);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm(1,0,3,2)
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm(2,3,0,1)
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));   // row_mirror
  return max(max(rows_u32(v, 0), rows_u32(v, 1)), max(rows_u32(v, 2), rows_u32(v, 3)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  return min(min(rows_u32(v, 0), rows_u32(v, 1)), min(rows_u32(v, 2), rows_u32(v, 3)));
}
// Order-preserving key of a float that is not NaN: a > b exactly when key(a) > key(b) (-0 is
// turned into +0 first, so equal values have equal keys).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Score sources. get4(t, lane, s, b) fills, for the lane's experts e = lane + 64 j (j < 4, e < E),
// s = sigmoid(logit) and b = s + bias[e].
struct ScoresFromPairs {   // (s, b) pairs written by the logits kernel, [T][E]
  const float2* sb;
  int E;
  __device__ void get4(int64_t t, int lane, float* s, float* b) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E) {
        const float2 p = sb[t * E + e];
        s[j] = p.x;
        b[j] = p.y;
      }
    }
  }
};
// KS partial logits [KS][T][E] (split over the hidden dimension), summed in chunk order. Loads go
// out 4 chunks x 4 experts at a time, unconditionally (indices past the end re-read the last valid
// element and are discarded), so they overlap instead of waiting one by one.
constexpr int kMaxChunks = 32;
struct ScoresFromPartials {
  const float* part;
  const float* bias;
  int KS;
  int64_t T;
  int E;
  __device__ void get4(int64_t t, int lane, float* s, float* b) const {
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t base[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) base[j] = t * E + min(lane + 64 * j, E - 1);
    const int64_t chunk = T * E;
    constexpr int BATCH = 8;
    for (int q0 = 0; q0 < KS; q0 += BATCH) {
      float v[BATCH][4];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t off = (int64_t)min(q0 + u, KS - 1) * chunk;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[u][j] = part[off + base[j]];
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (q0 + u < KS) z[j] = (q0 + u == 0) ? v[u][j] : z[j] + v[u][j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e >= E) continue;
      s[j] = 1.0f / (1.0f + expf(-z[j]));
      b[j] = s[j] + bias[e];
    }
  }
};

// Selects token t with the calling wave (all 64 lanes). bl: 256 floats and gsc: 64 floats of LDS
// private to the wave. Lanes k < K receive the k-th chosen expert and its weight: K rounds of a
// wave-wide argmax over the kept groups' experts, ordered by (b desc, index asc).
template <class Src>
__device__ __forceinline__ void select_token(const Src& src, int64_t t, int lane, float* bl,
                                             float* gsc, int E, int G, int Gk, int K, float scale,
                                             int& out_id, float& out_w) {
  const int gs = E / G;
  float sv[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  src.get4(t, lane, sv, bv);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) bl[e] = bv[j];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  // group score: sum of the two largest b of the group (duplicates count twice)
  float myscore = -INFINITY;
  if (lane < G) {
    float v1 = -INFINITY, v2 = -INFINITY;
#pragma unroll 8
    for (int m = 0; m < gs; ++m) {
      const float v = bl[lane * gs + m];
      if (v > v1) {
        v2 = v1;
        v1 = v;
      } else if (v > v2) {
        v2 = v;
      }
    }
    myscore = gs >= 2 ? v1 + v2 : v1;
    gsc[lane] = myscore;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  bool kept_me = false;
  if (lane < G) {
    int rank = 0;
    for (int q = 0; q < G; ++q) {
      const float o = gsc[q];
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
    // the largest value, then the lowest expert index among the lanes holding it
    const uint32_t key = order_key(v);
    const uint32_t kmax = wave_max_u32(key);
    e = (int)wave_min_u32(key == kmax ? (uint32_t)e : 0xFFFFFFFFu);
    // every lane now holds the winner e; its owner retires it
    const int owner = e & 63, slotj = e >> 6;
    float s_mine = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j == slotj) s_mine = sv[j];
    const float s_win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_mine), owner));
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
  out_id = my_id;
  out_w = scale * my_s / ssum;
  // the wave's LDS scratch is reused by its next token
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
}

}  // namespace beam
