/*
 * beam_moe.h — C ABI of the Beam routed-MoE block on AMD Instinct MI355X (gfx950).
 *
 * The block (sources, cited by tag and section):
 *   [S] "SGLang 原生支持 Reflection 的 Beam 并驱动其生产 API" (SGLang day-0 post for Beam)
 *   [V] "vLLM 实现 Reflection Beam 501B MoE 模型 Day 0 支持" (vLLM day-0 post for Beam)
 *   [H] "Reflection 发布 501B 开源模型 Beam，Apache 2.0 许可" (translated HF launch post)
 *   1. FP32 router: logits = x . W_r^T with FP32 weights, accumulation and logits
 *      ([V] §MoE and residual stream; [S] §Dense Layers and Grouped MoE Routing).
 *   2. Sigmoid scores plus an expert correction bias choose the experts; group-limited selection:
 *      G groups, group score = sum of its two largest biased scores, keep the best Gk groups, take
 *      the top K experts over their union ([V] ibid.; [H] §专家混合).
 *   3. Weights: the chosen experts' unbiased scores renormalised and multiplied by the routed
 *      scale (2.5 for Beam), kept in FP32 ([V] ibid.; [S] ibid.).
 *   4. K SwiGLU experts per token (hidden -> d_ff -> hidden, no biases) ([H] §专家混合), with the
 *      bf16 rounding points of the BF16 expert kernels: gate/up outputs and the activation product
 *      rounded to bf16, the FP32 routing weight applied to the down output before any rounding
 *      ([S] §BF16 MoE Kernel Optimization).
 *   5. Weighted combine over the K experts, no shared expert ([V] ibid.; [H] §专家混合).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and contiguous, with the
 *     base address 16-byte aligned. Inputs are never written. Outputs and the workspace are fully
 *     overwritten (plain stores, never accumulation).
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call is asynchronous on it; none
 *     allocates device memory, frees, or synchronises the host (except under BEAM_MOE_SYNC_CHECK).
 *   - Every argument is validated on the host before the first launch: a non-zero status means
 *     nothing was launched. T = 0 is a successful no-op. Device-side faults surface at the caller's
 *     next synchronisation. Unsupported shapes or dtypes return BEAM_ERR_UNSUPPORTED: there is no
 *     fallback path.
 *   - Calls on distinct workspaces may run concurrently on different streams; calls that share a
 *     workspace must be ordered by the caller.
 *   - Debugging: with the environment variable BEAM_MOE_SYNC_CHECK set to anything but "0" (read
 *     at the first launch) every launch is followed by a synchronisation of its stream, and a kernel
 *     that failed is reported on stderr, naming its stage, and returned as BEAM_ERR_LAUNCH by the
 *     call that launched it. This serialises the host with the GPU; not for use under stream
 *     capture.
 *   - NaN or infinite inputs give undefined (but memory-safe) results.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define BEAM_API __attribute__((visibility("default")))
#else
#define BEAM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t beam_status_t;

enum {
  BEAM_OK = 0,
  BEAM_ERR_NULL = 1,        /* a required pointer is NULL                                     */
  BEAM_ERR_ALIGN = 2,       /* a pointer is not 16-byte aligned                               */
  BEAM_ERR_SHAPE = 3,       /* T < 0, or dimensions inconsistent (e.g. E % G != 0, K > Gk*E/G) */
  BEAM_ERR_DTYPE = 4,       /* unknown dtype code, or a combination the block does not define */
  BEAM_ERR_UNSUPPORTED = 5, /* valid but not implemented for this shape (see the limits below) */
  BEAM_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace_bytes() figure  */
  BEAM_ERR_ALIAS = 7,       /* an output overlaps an input or another output                  */
  BEAM_ERR_LAUNCH = 8,      /* a kernel launch failed (the HIP error is reported by the runtime) */
  BEAM_ERR_DEVICE = 9       /* no usable gfx950 device is current                             */
};

/* dtype codes */
enum { BEAM_F32 = 0, BEAM_BF16 = 1, BEAM_FP8_E4M3 = 2 };

/* Shape and numerics of one MoE layer.
 *   hidden       H   model width (Beam 5120)
 *   n_experts    E   routed experts (Beam 256)
 *   n_groups     G   expert groups, contiguous, E/G experts each (Beam 8)
 *   topk_groups  Gk  groups kept per token (Beam 4)
 *   topk         K   experts per token (Beam 8)
 *   d_ff         F   expert intermediate width (Beam 2560)
 *   routed_scale     factor folded into the routing weights, so they sum to it (Beam 2.5)
 *   x_dtype      BEAM_BF16 or BEAM_F32 (token activations)
 *   w_dtype      BEAM_BF16, BEAM_FP8_E4M3 (with per-output-channel FP32 scales) or BEAM_F32 (expert
 *                weights). BEAM_F32 experts require x_dtype BEAM_F32 and compute without any rounding
 *                point; BEAM_BF16 / BEAM_FP8_E4M3 experts require x_dtype BEAM_BF16.
 *   out_dtype    BEAM_F32 (graded output) or BEAM_BF16 (round-to-nearest-even copy)
 * Limits of this library version: H % 256 == 0, F % 256 == 0, E <= 256, E % 16 == 0 and (E <= 64 or
 * E % 64 == 0), K <= 16, G <= 64, H * F < 2^31, T * K < 2^31; calls that run the experts on
 * BEAM_BF16 activations also need T * H < 2^31 (x under 4 GiB). */
typedef struct beam_moe_cfg {
  int32_t hidden;
  int32_t n_experts;
  int32_t n_groups;
  int32_t topk_groups;
  int32_t topk;
  int32_t d_ff;
  float routed_scale;
  int32_t x_dtype;
  int32_t w_dtype;
  int32_t out_dtype;
} beam_moe_cfg;

/* Routing only (steps 1–3).
 *   x         [T][H] x_dtype
 *   w_router  [E][H] fp32 — row e is expert e's router vector (the transpose of the H x E matrix)
 *   bias      [E] fp32 correction bias (selection only; it never enters the weights)
 *   topk_ids  [T][K] int32 out — chosen experts, biased score descending, ties to the lower id
 *   topk_w    [T][K] fp32 out — routed_scale * s_k / sum_j s_j, s = sigmoid(logit) (unbiased)
 *   workspace device scratch of at least beam_moe_route_workspace_bytes(cfg, T) bytes
 * Ties between equal FP32 scores (groups or experts) go to the lower index.
 * Logits are FP32 sums of exact products. With bf16 x and T > 1024 each FP32 router weight is split
 * exactly into three bf16 terms (valid for |w| >= 2^-102; smaller weights lose only bits below
 * 2^-126), written to the workspace, and the bf16 matrix cores accumulate the products in FP32;
 * otherwise the FP32 matrix cores multiply x (widened to FP32 if bf16) by the weights directly. */
BEAM_API beam_status_t beam_moe_route(const void* x, const float* w_router, const float* bias,
                             int32_t* topk_ids, float* topk_w, int64_t T,
                             const beam_moe_cfg* cfg, void* workspace, size_t workspace_bytes,
                             void* stream);
BEAM_API size_t beam_moe_route_workspace_bytes(const beam_moe_cfg* cfg, int64_t T);

/* The whole block (steps 1–5).
 *   x, w_router, bias      as for beam_moe_route
 *   w_gate_up  [E][2F][H] w_dtype — rows [0, F) are the gate projection, rows [F, 2F) the up
 *              projection; each row runs along H
 *   w_down     [E][H][F]  w_dtype — each row runs along F
 *   out        [T][H] out_dtype: out[t] = sum_k topk_w[t][k] * expert_{ids[t][k]}(x[t]), summed in
 *              k order in FP32
 *   w_gate_up_scale [E][2F], w_down_scale [E][H]: FP32 per-output-channel dequantisation scales
 *              for BEAM_FP8_E4M3 weights; must be NULL otherwise. With FP8 weights the activations
 *              are quantised on the fly: x per token and the intermediate h per row, each with
 *              scale amax/448, codes rounded to nearest-even and saturated to +-448.
 *   topk_ids_out [T][K] int32, topk_w_out [T][K] fp32: optional (NULL allowed) copies of the routing
 *   workspace  device scratch of at least beam_moe_workspace_bytes(cfg, T) bytes */
BEAM_API beam_status_t beam_moe_forward(const void* x, const float* w_router, const float* bias,
                               const void* w_gate_up, const void* w_down, void* out, int64_t T,
                               const beam_moe_cfg* cfg, const float* w_gate_up_scale,
                               const float* w_down_scale, int32_t* topk_ids_out,
                               float* topk_w_out, void* workspace, size_t workspace_bytes,
                               void* stream);
BEAM_API size_t beam_moe_workspace_bytes(const beam_moe_cfg* cfg, int64_t T);

/* beam_moe_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * workspace is a 64 MiB array of device memory the library holds per GPU until the process ends
 * (enough for beam_moe_workspace_bytes(cfg, T) <= 64 MiB: Beam's shape up to 327 tokens with bf16
 * experts, 290 with FP8 ones). The call
 * itself allocates nothing and leaves no state that a later call depends on.
 *   Arguments and results as for beam_moe_forward, without workspace / workspace_bytes.
 *   BEAM_ERR_WORKSPACE: beam_moe_workspace_bytes(cfg, T) exceeds 64 MiB (nothing is launched).
 * Every call on one GPU uses that GPU's one array: calls that may overlap on one GPU (different
 * streams, host threads) race and must be ordered by the caller. */
BEAM_API beam_status_t beam_moe_forward_noalloc(const void* x, const float* w_router,
                                                const float* bias, const void* w_gate_up,
                                                const void* w_down, void* out, int64_t T,
                                                const beam_moe_cfg* cfg,
                                                const float* w_gate_up_scale,
                                                const float* w_down_scale, int32_t* topk_ids_out,
                                                float* topk_w_out, void* stream);

/* Steps 4-5 with given routes, over a range of experts (routing replay and the expert-parallel
 * entry point: the routes are recorded once and reused instead of recomputed, so near-tied router
 * scores cannot pick a different expert path, [S] §Reinforcement learning in Miles; an expert-
 * parallel rank receives explicit expert ids and routing weights and runs its own experts,
 * including ranks with no local tokens, [S] §Fusion Optimizations).
 *   x          [T][H] x_dtype (as for beam_moe_forward)
 *   topk_ids   [T][K] int32: expert ids of each token's slots, as beam_moe_route writes them. Ids
 *              outside [expert_begin, expert_end) (including ids outside [0, E)) are skipped. Ids of
 *              one token must be distinct; a repeated id gives that token an unspecified (but
 *              memory-safe) output.
 *   topk_w     [T][K] fp32 routing weights, used as given (no renormalisation, no routed_scale)
 *   expert_begin, expert_end  the local experts, 0 <= expert_begin <= expert_end <= E
 *   w_gate_up  [expert_end - expert_begin][2F][H] w_dtype: the local experts' weights, local expert
 *              i being expert expert_begin + i (layout per expert as for beam_moe_forward)
 *   w_down     [expert_end - expert_begin][H][F] w_dtype
 *   w_gate_up_scale [expert_end - expert_begin][2F], w_down_scale [expert_end - expert_begin][H]:
 *              FP8 only, as for beam_moe_forward (NULL otherwise)
 *   With an empty range (expert_begin == expert_end) the weight and scale pointers may be NULL.
 *   out        [T][H] out_dtype: out[t] = sum, in k order from +0, over the slots k whose id e lies in
 *              the range, of topk_w[t][k] * expert_e(x[t]). Tokens without such slots get zeros. With
 *              the full range [0, E) and the routes of beam_moe_route this equals beam_moe_forward;
 *              summing the outputs of a partition of [0, E) gives it up to FP32 reassociation.
 *   workspace  device scratch of at least beam_moe_workspace_bytes(cfg, T) bytes
 * Validation and errors as for beam_moe_forward; a bad range is BEAM_ERR_SHAPE. */
BEAM_API beam_status_t beam_moe_forward_routed(const void* x, const int32_t* topk_ids,
                                               const float* topk_w, const void* w_gate_up,
                                               const void* w_down, void* out, int64_t T,
                                               const beam_moe_cfg* cfg, int32_t expert_begin,
                                               int32_t expert_end, const float* w_gate_up_scale,
                                               const float* w_down_scale, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* A dense SwiGLU MLP layer (Beam's first three layers are dense, d_ff 20480: [V] §MoE and residual
 * stream; [H] §专家混合), computed by the same grouped kernels as one expert that every token is
 * routed to with weight 1, under the same numerics contract (gate/up outputs and the activation
 * product rounded to bf16, the down projection in FP32).
 *   x          [T][hidden] bf16
 *   w_gate_up  [2 d_ff][hidden] w_dtype (BEAM_BF16 or BEAM_FP8_E4M3): rows [0, d_ff) gate, the rest up
 *   w_down     [hidden][d_ff] w_dtype
 *   out        [T][hidden] out_dtype (BEAM_F32 or BEAM_BF16): down(silu(gate x) * up x)
 *   w_gate_up_scale [2 d_ff], w_down_scale [hidden]: FP32 per-output-channel scales for FP8 weights
 *              (activations then quantised on the fly as in beam_moe_forward); NULL otherwise
 *   workspace  device scratch of at least beam_dense_mlp_workspace_bytes(hidden, d_ff, w_dtype, T)
 * Limits: hidden % 256 == 0, d_ff % 256 == 0, hidden * d_ff < 2^31, T * hidden < 2^31. Errors as
 * for beam_moe_forward. */
BEAM_API beam_status_t beam_dense_mlp_forward(const void* x, const void* w_gate_up,
                                              const void* w_down, void* out, int64_t T,
                                              int32_t hidden, int32_t d_ff, int32_t w_dtype,
                                              int32_t out_dtype, const float* w_gate_up_scale,
                                              const float* w_down_scale, void* workspace,
                                              size_t workspace_bytes, void* stream);
BEAM_API size_t beam_dense_mlp_workspace_bytes(int32_t hidden, int32_t d_ff, int32_t w_dtype,
                                               int64_t T);

/* Sublayer boundary: output RMSNorm of a sublayer, depth-scaled residual add, and the next sublayer's
 * input RMSNorm, in one pass (sandwich norm and depth-scaled residuals: [V] §MoE and residual stream;
 * the fused norm -> residual -> norm transition with FP32 math and bf16 rounding points: [V]
 * §Agent-driven optimization item 1, [S] §Sandwich Normalization and Depth-Scaled Residuals;
 * [H] §残差流). Per token, FP32 arithmetic, each rounding to bf16 marked bf16():
 *   u  = bf16(y)                                      (the sublayer output in the activation dtype)
 *   p  = bf16(u * gamma_post / sqrt(mean(u^2) + eps))
 *   h' = bf16(bf16(sqrt((n-1)/n) * h) + bf16(p / sqrt(n)))      n = depth_n >= 1
 *   x' = bf16(h' * gamma_next / sqrt(mean(h'^2) + eps))
 *   y          [T][hidden] y_dtype (BEAM_F32 or BEAM_BF16): the sublayer output
 *   h          [T][hidden] bf16: the residual stream before the add
 *   gamma_post, gamma_next  [hidden] fp32 RMSNorm weights (output norm of this sublayer, input norm
 *              of the next one)
 *   h_out      [T][hidden] bf16 out: h'. May be h itself (in place); no other overlap.
 *   x_next     [T][hidden] bf16 out: x'
 *   depth_n    the residual add's index n (the input embedding counts as add 1)
 *   eps        RMSNorm epsilon (>= 0; the pages do not state it)
 * Limits: hidden % 256 == 0, hidden <= 16384. */
BEAM_API beam_status_t beam_residual_boundary(const void* y, int32_t y_dtype, const void* h,
                                              const float* gamma_post, const float* gamma_next,
                                              void* h_out, void* x_next, int64_t T,
                                              int32_t hidden, int32_t depth_n, float eps,
                                              void* stream);

/* beam_moe_forward with its combine fused into the boundary that follows the MoE sublayer (after the
 * MoE the boundary kernel also combines the top-k expert outputs: [V] §Agent-driven optimization
 * item 3): y is the FP32 combine of the routed experts (as `out` of beam_moe_forward), and the
 * boundary above is applied to it. Arguments as for beam_moe_forward (x_dtype must be BEAM_BF16;
 * out_dtype is unused) and beam_residual_boundary. */
BEAM_API beam_status_t beam_moe_forward_boundary(
    const void* x, const float* w_router, const float* bias, const void* w_gate_up,
    const void* w_down, int64_t T, const beam_moe_cfg* cfg, const float* w_gate_up_scale,
    const float* w_down_scale, const void* h, const float* gamma_post, const float* gamma_next,
    int32_t depth_n, float eps, void* h_out, void* x_next, int32_t* topk_ids_out, float* topk_w_out,
    void* workspace, size_t workspace_bytes, void* stream);

/* Dynamic FP8 E4M3 quantisation of bf16 rows, the activation step of the FP8 experts (dynamic FP8
 * checkpoints: [S] §Highlights, §BF16, NVFP4 and FP8 Model Support).
 *   src    [rows][cols] bf16 (device), cols % 8 == 0
 *   codes  [rows][cols] uint8 out: OCP E4M3FN codes of v * (448 / amax_row), rounded to nearest even
 *          and saturated to +-448; the sign of zero follows the input
 *   scales [rows] fp32 out: amax_row / 448 (1 for an all-zero row, whose codes are all 0)
 * amax, the scale and the product are taken in FP32 with correctly rounded operations. */
BEAM_API beam_status_t beam_moe_quant_fp8(const void* src, int64_t rows, int32_t cols,
                                          uint8_t* codes, float* scales, void* stream);

/* Element conversion with the rounding routines of the kernels (the bf16 rounding points of the
 * expert path, [S] §BF16 MoE Kernel Optimization; the E4M3 codes of the dynamic FP8 path, [S] §BF16,
 * NVFP4 and FP8 Model Support), for checking them and for preparing inputs.
 *   src  [n] fp32 (device); finite values
 *   dst  [n] out: dst_dtype BEAM_BF16 -> bf16 bits rounded to nearest even (values past the largest
 *        bf16 and NaN inputs are unspecified); BEAM_FP8_E4M3 -> OCP E4M3FN codes rounded to nearest
 *        even and saturated to +-448, the sign of zero kept */
BEAM_API beam_status_t beam_moe_convert(const float* src, int64_t n, int32_t dst_dtype, void* dst,
                                        void* stream);

/* The FP8 matrix instruction of the FP8 expert GEMMs on caller tiles, for checking its summation:
 * per tile t, d[t] = a[t] . b[t]^T + c[t] with one 16x16x128 E4M3 MFMA (unit block scales), the sum
 * taken by the instruction itself (it does not round each partial sum to FP32: its result can differ
 * from the FP32 rounding of the exact sum by a few 1e-4 of the largest |product|).
 *   a, b  [n_tiles][16][128] uint8 E4M3 codes (rows along the 128-deep contraction)
 *   c, d  [n_tiles][16][16] fp32 (d[t][i][j] = sum_k a[t][i][k] b[t][j][k] + c[t][i][j]) */
BEAM_API beam_status_t beam_moe_fp8_dot_tiles(const uint8_t* a, const uint8_t* b, const float* c,
                                              float* d, int64_t n_tiles, void* stream);

/* Inspection of a forward's intermediate arrays, for tests and debugging. After a call of
 * beam_moe_forward or beam_moe_forward_routed with the same cfg and T has completed on `workspace`,
 * the bytes [*offset, *offset + *bytes) of that workspace hold the array named by `region`:
 *   BEAM_WS_EXPERT_OFF  int32 [n + 1]  first sorted row of each of the call's n experts (n = E for
 *                       beam_moe_forward, expert_end - expert_begin for the routed call); entry n
 *                       is the number of sorted rows
 *   BEAM_WS_SORTED_SLOT int32 [T*K]    slot t*K + k of each sorted row (rows of one expert are
 *                       contiguous and in token order)
 *   BEAM_WS_H           [T*K][F]       the expert activation h of each sorted row (bf16; fp32 for
 *                       BEAM_F32 experts), after its rounding point
 *   BEAM_WS_HQ, BEAM_WS_HS  (BEAM_FP8_E4M3 only) uint8 [T*K][F] E4M3 codes and fp32 [T*K] scales
 *                       of the h rows, as the down GEMM consumes them
 *   BEAM_WS_XQ, BEAM_WS_XS  (BEAM_FP8_E4M3 only) uint8 [T][H] E4M3 codes and fp32 [T] scales of x
 *   BEAM_WS_Y           fp32 [T*K][H]  the weighted output topk_w * y of each slot (indexed by slot;
 *                       slots routed outside the call's experts hold stale values)
 * Rows past the number of sorted rows hold stale values. Returns BEAM_ERR_SHAPE / _UNSUPPORTED /
 * _DTYPE as beam_moe_workspace_bytes would fail, BEAM_ERR_NULL for NULL outputs and
 * BEAM_ERR_UNSUPPORTED for a region the cfg does not have (e.g. HQ without FP8 experts). No
 * device work is done. */
enum {
  BEAM_WS_EXPERT_OFF = 0,
  BEAM_WS_SORTED_SLOT = 1,
  BEAM_WS_H = 2,
  BEAM_WS_HQ = 3,
  BEAM_WS_HS = 4,
  BEAM_WS_XQ = 5,
  BEAM_WS_XS = 6,
  BEAM_WS_Y = 7
};
BEAM_API beam_status_t beam_moe_workspace_region(const beam_moe_cfg* cfg, int64_t T, int32_t region,
                                                 size_t* offset, size_t* bytes);
/* The same for a beam_dense_mlp_forward workspace (one expert that every token takes with weight 1:
 * K = 1, n = 1). There BEAM_WS_Y is sized for up to four partial rows per token: a call whose down
 * GEMM splits its K range into p parts writes row t*p + i with part i, summed in part order by the
 * combine (p is chosen per call from the shape and the device and is not reported). */
BEAM_API beam_status_t beam_dense_mlp_workspace_region(int32_t hidden, int32_t d_ff,
                                                       int32_t w_dtype, int64_t T, int32_t region,
                                                       size_t* offset, size_t* bytes);

/* Human-readable name of a status code (static storage, never NULL). */
BEAM_API const char* beam_status_string(beam_status_t status);

/* Library version as major * 10000 + minor * 100 + patch. */
BEAM_API int32_t beam_moe_version(void);

/* Per-stage timing for measurement (not thread-safe; off by default).
 * beam_moe_timing_enable(1) makes later forward/route calls record a HIP event pair around each
 * stage on the call's stream; beam_moe_timing_collect() synchronises those events, writes per-stage
 * totals (milliseconds) and launch counts for up to n_stages stages, releases the events and
 * returns the number of stages defined. Stage order: 0 router logits, 1 router select,
 * 2 moe_align, 3 activation quant (fp8), 4 gate/up GEMM, 5 h quant (fp8), 6 down GEMM,
 * 7 combine (for forwards of up to 16 tokens the selection and the align are one launch, recorded
 * as stage 1; past 1024 tokens with bf16 activations the logits and the selection are one launch,
 * recorded as stage 0 together with the split of the router weights that precedes it). beam_moe_stage_name(i) names stage i.
 * beam_moe_timing_stages(mask) restricts the recording to the stages whose bit (1 << stage) is set
 * (default: all), so a caller can time one kernel without event records between the others. */
BEAM_API void beam_moe_timing_enable(int32_t enable);
BEAM_API void beam_moe_timing_stages(uint32_t stage_mask);
BEAM_API int32_t beam_moe_timing_collect(double* total_ms, int32_t* launches, int32_t n_stages);
BEAM_API const char* beam_moe_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_MOE_H */
