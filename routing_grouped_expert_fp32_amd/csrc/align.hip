// moe_align: group the T*K routed slots by expert for the grouped GEMMs (gfx950).
//
// The TRTLLM MoE path the vLLM post lists ([V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持"
// §The fused graph) has routing/permutation kernels between the router and the grouped GEMMs; this
// is that step, designed for wave64:
//   1. align_count   (one WG per chunk of 256 tokens): per expert, a 256-bit mask of which tokens
//                    of the chunk chose it (LDS 64-bit atomic OR); popcounts give chunk counts.
//   2. align_scan    (one WG of 1024 threads): per expert, exclusive prefix over chunks, expert
//                    totals and offsets, and the row-block table: an expert with c rows gets
//                    floor(c/BM) full blocks of BM rows and one block with the remainder, so
//                    skewed experts split into many full blocks and only the last block of an
//                    expert is partly filled (the GEMMs skip its empty 16-row sub-tiles).
//   3. align_scatter (one WG per chunk): each slot's row = expert offset + chunk base + number of
//                    earlier tokens of the chunk that chose the same expert (popcount of the mask
//                    below the token's bit). Rows of an expert are therefore in token order — a
//                    deterministic, stable permutation; no sort, no global atomics.
// Only the experts [e_begin, e_begin + E) take part (the forward uses all of them; a routed call
// may restrict itself to a local range): slots naming any other id are left out, and expert
// indices in the tables are local (id - e_begin), so the GEMMs index a local weight array.
// Slots of one token name distinct experts (the router guarantees it; for given routes a repeated
// id within a token leaves one of its slots out, which is memory-safe).
#include "device_common.h"
#include "route_select.h"

namespace beam {

constexpr int kChunk = kAlignChunk;
constexpr int kWords = kAlignWords;

__global__ __launch_bounds__(256) void align_count_kernel(const int32_t* __restrict__ ids,
                                                          uint64_t* __restrict__ chunk_mask,
                                                          int32_t* __restrict__ chunk_cnt,
                                                          int64_t T, int E, int K, int e_begin) {
  __shared__ unsigned long long mask[256 * kWords];
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < E * kWords; i += 256) mask[i] = 0ull;
  __syncthreads();
  const int64_t tbeg = (int64_t)c * kChunk;
  const int ntok = (int)((T - tbeg) < kChunk ? (T - tbeg) : kChunk);
  const int nslot = ntok * K;
  for (int i = threadIdx.x; i < nslot; i += 256) {
    const int tl = i / K;
    const int e = ids[tbeg * K + i] - e_begin;
    if ((unsigned)e >= (unsigned)E) continue;   // not one of this call's experts
    atomicOr(&mask[e * kWords + (tl >> 6)], 1ull << (tl & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      const uint64_t m = mask[e * kWords + w];
      chunk_mask[((int64_t)c * E + e) * kWords + w] = m;
      cnt += __popcll(m);
    }
    chunk_cnt[(int64_t)c * E + e] = cnt;
  }
}

// 1024 threads: 4 segments of the chunk range x 256 experts.
__global__ __launch_bounds__(1024) void align_scan_kernel(int32_t* __restrict__ chunk_base,
                                                          int32_t* __restrict__ expert_count,
                                                          int32_t* __restrict__ expert_off,
                                                          int32_t* __restrict__ n_blocks,
                                                          int32_t* __restrict__ blk_expert,
                                                          int32_t* __restrict__ blk_row0,
                                                          int32_t* __restrict__ blk_rows,
                                                          int n_chunks, int E, int BM) {
  __shared__ int seg_sum[4][256];
  __shared__ int scan_rows[256];
  __shared__ int scan_blks[256];
  const int e = threadIdx.x & 255, seg = threadIdx.x >> 8;
  const int per = (n_chunks + 3) / 4;
  const int cb = seg * per, ce = min(n_chunks, cb + per);
  // pass 1: segment totals (independent loads, unrolled so many are in flight)
  int sum = 0;
  if (e < E) {
    int c = cb;
    for (; c + 8 <= ce; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = chunk_base[(int64_t)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; c < ce; ++c) sum += chunk_base[(int64_t)c * E + e];
  }
  seg_sum[seg][e] = sum;
  __syncthreads();
  // pass 2: exclusive prefix over chunks, in place (counts -> bases)
  if (e < E) {
    int run = 0;
    for (int q = 0; q < seg; ++q) run += seg_sum[q][e];
    int c = cb;
    for (; c + 8 <= ce; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = chunk_base[(int64_t)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        chunk_base[(int64_t)(c + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; c < ce; ++c) {
      const int v = chunk_base[(int64_t)c * E + e];
      chunk_base[(int64_t)c * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  // expert totals, offsets and block counts: exclusive scans over experts (threads 0..255)
  int count = 0, nb = 0;
  if (seg == 0) {
    if (e < E) count = seg_sum[0][e] + seg_sum[1][e] + seg_sum[2][e] + seg_sum[3][e];
    nb = (count + BM - 1) / BM;
    scan_rows[e] = count;
    scan_blks[e] = nb;
  }
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int vr = 0, vb = 0;
    if (seg == 0 && e >= off) {
      vr = scan_rows[e - off];
      vb = scan_blks[e - off];
    }
    __syncthreads();
    if (seg == 0 && e >= off) {
      scan_rows[e] += vr;
      scan_blks[e] += vb;
    }
    __syncthreads();
  }
  if (seg == 0 && e < E) {
    const int row_start = scan_rows[e] - count;   // inclusive -> exclusive
    const int blk_start = scan_blks[e] - nb;
    expert_count[e] = count;
    expert_off[e] = row_start;
    if (e == E - 1) {
      expert_off[E] = scan_rows[e];
      n_blocks[0] = scan_blks[e];
    }
    for (int i = 0; i < nb; ++i) {   // full blocks of BM rows, then the remainder
      blk_expert[blk_start + i] = e;
      blk_row0[blk_start + i] = row_start + i * BM;
      blk_rows[blk_start + i] = min(BM, count - i * BM);
    }
  }
}

__global__ __launch_bounds__(256) void align_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const uint64_t* __restrict__ chunk_mask,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ expert_off,
                                                            const float* __restrict__ topk_w,
                                                            int32_t* __restrict__ sorted_slot,
                                                            float* __restrict__ sorted_w,
                                                            int64_t T, int E, int K, int e_begin) {
  __shared__ unsigned long long mask[256 * kWords];
  __shared__ int base[256];
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < E * kWords; i += 256)
    mask[i] = chunk_mask[(int64_t)c * E * kWords + i];
  for (int e = threadIdx.x; e < E; e += 256)
    base[e] = expert_off[e] + chunk_base[(int64_t)c * E + e];
  __syncthreads();
  const int64_t tbeg = (int64_t)c * kChunk;
  const int ntok = (int)((T - tbeg) < kChunk ? (T - tbeg) : kChunk);
  const int nslot = ntok * K;
  for (int i = threadIdx.x; i < nslot; i += 256) {
    const int tl = i / K;
    const int e = ids[tbeg * K + i] - e_begin;
    if ((unsigned)e >= (unsigned)E) continue;
    const int w = tl >> 6;
    int rank = 0;
    for (int q = 0; q < w; ++q) rank += __popcll(mask[e * kWords + q]);
    const uint64_t below = (tl & 63) ? (mask[e * kWords + w] & ((1ull << (tl & 63)) - 1ull)) : 0ull;
    rank += __popcll(below);
    sorted_slot[base[e] + rank] = (int32_t)(tbeg * K + i);
    sorted_w[base[e] + rank] = topk_w[tbeg * K + i];
  }
}

// ---------------------------------------------------------------------------------------------
// Small batches (T <= kSmallAlignT = 64 tokens): the whole align in one workgroup of 1024 threads.
// One 64-bit mask per expert (bit t: token t chose it), counts by popcount, exclusive scans over the
// experts in LDS, the same block table and the same stable token order as the three-kernel path.
static_assert(kSmallAlignT <= 64, "one mask word per expert");

__device__ void align_small_body(const int32_t* sid, const float* tw, int64_t T, int E, int K,
                                 int e_begin, int BM, const AlignTables& at) {
  __shared__ unsigned long long mask[256];
  __shared__ int rows_scan[256];
  __shared__ int blks_scan[256];
  const int tid = threadIdx.x;
  if (tid < 256) mask[tid] = 0ull;
  __syncthreads();
  const int nslot = (int)T * K;
  for (int i = tid; i < nslot; i += blockDim.x) {
    const int e = sid[i] - e_begin;
    if ((unsigned)e < (unsigned)E) atomicOr(&mask[e], 1ull << (i / K));
  }
  __syncthreads();
  int count = 0, nb = 0;
  if (tid < 256) {
    count = tid < E ? __popcll(mask[tid]) : 0;
    nb = (count + BM - 1) / BM;
    rows_scan[tid] = count;
    blks_scan[tid] = nb;
  }
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int vr = 0, vb = 0;
    if (tid < 256 && tid >= off) {
      vr = rows_scan[tid - off];
      vb = blks_scan[tid - off];
    }
    __syncthreads();
    if (tid < 256 && tid >= off) {
      rows_scan[tid] += vr;
      blks_scan[tid] += vb;
    }
    __syncthreads();
  }
  if (tid < E) {
    const int row_start = rows_scan[tid] - count;
    const int blk_start = blks_scan[tid] - nb;
    at.expert_count[tid] = count;
    at.expert_off[tid] = row_start;
    if (tid == E - 1) {
      at.expert_off[E] = rows_scan[tid];
      at.n_blocks[0] = blks_scan[tid];
    }
    for (int i = 0; i < nb; ++i) {   // full blocks of BM rows, then the remainder
      at.blk_expert[blk_start + i] = tid;
      at.blk_row0[blk_start + i] = row_start + i * BM;
      at.blk_rows[blk_start + i] = min(BM, count - i * BM);
    }
  }
  for (int i = tid; i < nslot; i += blockDim.x) {
    const int e = sid[i] - e_begin;
    if ((unsigned)e >= (unsigned)E) continue;
    const int t = i / K;
    const int rank = __popcll(mask[e] & ((1ull << t) - 1ull));
    at.sorted_slot[rows_scan[e] - __popcll(mask[e]) + rank] = i;
    at.sorted_w[rows_scan[e] - __popcll(mask[e]) + rank] = tw[i];
  }
}

__global__ __launch_bounds__(1024) void align_small_kernel(const int32_t* __restrict__ ids,
                                                           const float* __restrict__ tw,
                                                           AlignTables at, int64_t T, int E, int K,
                                                           int e_begin, int BM) {
  align_small_body(ids, tw, T, E, K, e_begin, BM, at);
}

// The smallest batches of the forward (up to 16 tokens): selection and align in one launch. One
// workgroup of 16 waves: wave w selects token w (select_token), writes its routes and keeps them in
// LDS, then the workgroup groups the slots by expert (align_small_body) from LDS. (With more tokens
// a single workgroup would select several tokens per wave one after another, slower than the
// selection over many workgroups plus a separate align launch.)
__global__ __launch_bounds__(1024) void select_align_small_kernel(ScoresFromPartials src,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ wout,
                                                                  AlignTables at, int64_t T, int E,
                                                                  int G, int Gk, int K, float scale,
                                                                  int BM) {
  __shared__ float bl[16][256];
  __shared__ float gsc[16][64];
  __shared__ int32_t sid[kSmallAlignT * 16];
  __shared__ float sw[kSmallAlignT * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t t = wave; t < T; t += 16) {
    int id;
    float w;
    select_token(src, t, lane, bl[wave], gsc[wave], E, G, Gk, K, scale, id, w);
    if (lane < K) {
      ids[t * K + lane] = id;
      wout[t * K + lane] = w;
      sid[t * K + lane] = id;
      sw[t * K + lane] = w;
    }
  }
  __syncthreads();
  align_small_body(sid, sw, T, E, K, 0, BM, at);
}

hipError_t launch_select_align_small(const float* part, const float* bias, int32_t* ids, float* w,
                                     const AlignTables& at, const Shape& s, int BM,
                                     hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (!use_fused_select_align(s)) return hipErrorInvalidValue;
  const ScoresFromPartials src{part, bias, router_partial_chunks(s), s.T, s.E};
  hipLaunchKernelGGL(select_align_small_kernel, dim3(1), dim3(1024), 0, st, src, ids, w, at, s.T,
                     s.E, s.G, s.Gk, s.K, s.scale, BM);
  return hipGetLastError();
}

// Routes of a dense layer run as one expert: every token's single slot goes to expert 0 with
// weight 1 (so the down epilogue and the combine are exact copies of the MLP output).
__global__ __launch_bounds__(256) void fill_dense_routes_kernel(int32_t* __restrict__ ids,
                                                                float* __restrict__ w, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    ids[i] = 0;
    w[i] = 1.0f;
  }
}

hipError_t launch_fill_dense_routes(int32_t* ids, float* w, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_dense_routes_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st,
                     ids, w, n);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* ids, const float* topk_w, const AlignTables& at,
                        const Shape& s, int BM, int e_begin, int e_count, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.T <= kSmallAlignT) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(1024), 0, st, ids, topk_w, at, s.T,
                       e_count, s.K, e_begin, BM);
    return hipGetLastError();
  }
  const int n_chunks = (int)ceil_div(s.T, kChunk);
  hipLaunchKernelGGL(align_count_kernel, dim3(n_chunks), dim3(256), 0, st, ids, at.chunk_mask,
                     at.chunk_base, s.T, e_count, s.K, e_begin);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, st, at.chunk_base,
                     at.expert_count, at.expert_off, at.n_blocks, at.blk_expert, at.blk_row0,
                     at.blk_rows, n_chunks, e_count, BM);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(n_chunks), dim3(256), 0, st, ids, at.chunk_mask,
                     at.chunk_base, at.expert_off, topk_w, at.sorted_slot, at.sorted_w, s.T,
                     e_count, s.K, e_begin);
  return hipGetLastError();
}

}  // namespace beam
