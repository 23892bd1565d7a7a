"""Benchmark of the Beam routed-MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                    [--also prefill,skew,fp8_decode,fp8_prefill,routed_prefill,
                            dense_prefill,boundary_prefill,small_t]
                    [--no-cpu-baseline]

A step is one beam_moe_forward over one batch (router, selection, moe_align, [FP8 quantisers],
gate/up GEMM, down GEMM, combine), inputs already resident in HBM. The timed region is bracketed by
torch.cuda.synchronize() on both sides; inside it the library records HIP events on the call's
stream around the gate/up GEMM only (the roofline kernel), which gives that kernel's average
duration without event records between the other kernels; stages_ms comes from a second,
instrumented pass of the same steps with every stage recorded, and its step_ms_p10_median_p90 from a
third pass with an event pair around every call. route_only_ms times beam_moe_route on its own.
Prints ONE JSON line; the
headline `value` is the --workload (decode, T=32, the configuration the metric is quoted on), the
other workloads are reported under "also". skew is the T=32768 batch whose correction bias puts
40% of the slots on 16 hot experts (about 6.5K rows each, MFMA-bound). routed_prefill / routed_decode time
beam_moe_forward_routed over one expert-parallel share (experts 32..63, one group) of that batch,
with the router's routes computed once beforehand; their bytes and FLOPs count the local slots and
experts only. dense_prefill times beam_dense_mlp_forward on Beam's dense layer (d_ff 20480) at
T=8192. boundary_prefill times beam_moe_forward_boundary (combine fused into the post-MoE
norm -> residual -> norm boundary) and the standalone boundary at T=8192. small_t times the
decode-shaped layer at T = 1, 2, 4, 8, 16 and 64 (no timing events inside the steps) against its HBM
floor: distinct experts touched x 78.6 MB of bf16 weights / 8 TB/s.

roofline (dominant kernel = the gate/up grouped GEMM). Algorithmic bytes per launch = distinct
experts touched (counted from the routing of the batch) x the expert's gate and up weights (bf16:
2*d_ff*hidden*2 B; FP8: 2*d_ff*hidden codes + 2*d_ff*4 B scales) + the token rows read once (bf16 x,
or FP8 codes + scales) + h written once (T*K*d_ff*2 B), divided by the kernel's average duration.
Each weight byte feeds one multiply-add per routed row (bf16: 2 FLOP / 2 B; FP8: 2 FLOP / 1 B), so
FLOP/B = T*K/E (bf16) or 2*T*K/E (FP8); below the ridge (bf16 2.5 PFLOP/s / 8 TB/s = 312; FP8
5.0 / 8 = 625) the bound is "hbm", else "mfma" with FLOP = 2*T*K*2*d_ff*hidden.
traffic: HBM bytes of that kernel from rocprofv3 --pmc runs (2.0 x FETCH_SIZE + WRITE_SIZE, the
factor from a 1 GiB copy), stored in profiles/counters_<workload>.json with a hash of the kernel
sources; null if the file is missing or the sources changed since.
ceilings: measured context for the fractions (vendor-library calls, not the measured path): a 4 GiB
device copy, an 8192^3 bf16 matmul and a dense batched bf16 GEMM of the prefill gate/up shape.
cpu_baseline: the CPU oracle (float64 numpy) on a bounded sample of the same batch (routing of the
whole batch + expert MLPs and combine for the first --cpu-tokens tokens), on the host's cores;
one_core: the same on one thread, experts of an eighth of the tokens.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
KERNEL_SOURCES = ("gemm_grouped.hip", "gemm_pipe.h", "gemm_small.h", "common.h",
                  "device_common.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "routing_grouped_expert_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "prefill", "skew", "fp8_decode", "fp8_prefill",
                            "routed_prefill", "routed_decode"])
    p.add_argument("--also", default="prefill,skew,fp8_decode,fp8_prefill,routed_prefill,"
                   "dense_prefill,boundary_prefill,small_t",
                   help="comma list of extra workloads ('' = none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured HBM / GEMM ceilings (vendor-library context)")
    p.add_argument("--cpu-tokens", type=int, default=32)
    p.add_argument("--copy-probe-gib", type=float, default=0.0,
                   help="also run a plain device copy of this size (counter scaling reference)")
    return p.parse_args()


def skew_delta():
    with open(os.path.join(ROOT, "tests", "golden", "skew_bias.json")) as f:
        return json.load(f)["delta"]


class Weights:
    """Beam expert weights on the GPU, generated once per dtype."""

    def __init__(self, synthgen, torch):
        self.sg, self.torch, self.cache = synthgen, torch, {}

    def get(self, w_dtype):
        if w_dtype not in self.cache:
            name = "fp8_prefill" if w_dtype == "fp8" else "prefill"
            print(f"[bench] generating Beam {w_dtype} expert weights", file=sys.stderr, flush=True)
            self.cache[w_dtype] = self.sg.make_inputs(name, device="cuda", T=1)
            self.torch.cuda.synchronize()
        return self.cache[w_dtype]


def timed_steps(bm, torch, step, steps, warmup, stage):
    """Warm up, then time `steps` calls with the wall clock while the library records HIP events
    around `stage` only (one event pair per call on the call's stream, so no event records sit
    between the other kernels); then a second, instrumented pass of the same calls records every
    stage for the breakdown. Returns (ms per step, average ms of `stage` in the timed steps,
    {stage: ms per step, summed over its launches} of the instrumented pass)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    bm.timing_enable(True, stages=[stage])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    bm.timing_enable(False)
    tot, cnt = bm.timing_collect()[stage]
    bm.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    bm.timing_enable(False)
    stages = {k: (v[0] / steps if v[1] else None) for k, v in bm.timing_collect().items()}
    # per-step spread: a third pass with an event pair around every call on the calling stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]  # noqa: E731
    stages["step_ms_p10_median_p90"] = [q(0.1), q(0.5), q(0.9)]
    return elapsed * 1e3 / steps, tot / max(cnt, 1), stages


# routed workloads: beam_moe_forward_routed over one expert-parallel share (one group of 32
# experts, as eight ranks would hold them) of a workload's batch, with the router's routes
ROUTED = {"routed_prefill": ("prefill", 32, 64), "routed_decode": ("decode", 32, 64)}


def measure(bm, synthgen, torch, name, weights, steps, warmup):
    routed = ROUTED.get(name)
    base = routed[0] if routed else name
    wl = synthgen.WORKLOADS[base]
    W = weights.get(wl.w_dtype)
    d = synthgen.make_inputs(wl, device="cuda", with_experts=False,
                             skew_delta=skew_delta() if base == "skew" else None)
    sh = wl.shape
    fp8 = wl.w_dtype == "fp8"
    cfg = bm.WorkloadCfg.of(sh, wl.x_dtype, wl.w_dtype)
    T = wl.T
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, sh.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, sh.topk), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    scales = dict(w_gate_up_scale=W.get("w_gate_up_scale"), w_down_scale=W.get("w_down_scale"))

    def step():
        bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg, out=out,
                   topk_ids_out=ids, workspace=ws, stream=stream, **scales)

    n_slots = T * sh.topk
    if routed:
        b, e = routed[1], routed[2]
        tw = torch.empty((T, sh.topk), dtype=torch.float32, device="cuda")
        bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg, out=out,
                   topk_ids_out=ids, topk_w_out=tw, workspace=ws, stream=stream, **scales)
        local = {k: (v[b:e] if v is not None else None) for k, v in scales.items()}
        wgu, wdn = W["w_gate_up"][b:e], W["w_down"][b:e]
        torch.cuda.synchronize()
        n_slots = int(((ids >= b) & (ids < e)).sum())

        def step():  # noqa: F811
            bm.forward_routed(d["x"], ids, tw, wgu, wdn, cfg, b, e, out=out, workspace=ws,
                              stream=stream, **local)

    ms, gu_ms, stages_ms = timed_steps(bm, torch, step, steps, warmup, "gate_up")
    route_ms = None
    if not routed:   # beam_moe_route on its own (router logits + selection)
        rws = torch.empty(max(bm.route_workspace_bytes(cfg, T), 16), dtype=torch.uint8,
                          device="cuda")
        rid = torch.empty((T, sh.topk), dtype=torch.int32, device="cuda")
        rw = torch.empty((T, sh.topk), dtype=torch.float32, device="cuda")
        rstep = lambda: bm.route(d["x"], W["w_router"], d["bias"], cfg, topk_ids=rid,  # noqa
                                 topk_w=rw, workspace=rws, stream=stream)
        for _ in range(warmup):
            rstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            rstep()
        torch.cuda.synchronize()
        route_ms = (time.perf_counter() - t0) * 1e3 / steps
        del rws
    u = torch.unique(ids)
    if routed:
        u = u[(u >= routed[1]) & (u < routed[2])]
    distinct = int(u.numel())
    F, H, K, E = sh.d_ff, sh.hidden, sh.topk, sh.n_experts
    if routed:
        E = routed[2] - routed[1]
    wb = 1 if fp8 else 2                                   # bytes per weight element
    gu_w = 2 * F * H * wb + (2 * F * 4 if fp8 else 0)      # gate+up bytes of one expert
    dn_w = H * F * wb + (H * 4 if fp8 else 0)
    x_bytes = T * H * (1 + 4.0 / H if fp8 else 2)
    gu_bytes = distinct * gu_w + x_bytes + n_slots * F * 2
    gu_flops = 2.0 * n_slots * 2 * F * H
    flop_per_byte = (2.0 if fp8 else 1.0) * n_slots / E
    dt = "fp8" if fp8 else "bf16"
    ridge = PEAK_TFLOPS[dt] * 1e12 / (HBM_PEAK_GBS * 1e9)
    router_bytes = 0 if routed else E * H * 4 + E * 4
    layer_bytes = distinct * (gu_w + dn_w) + router_bytes + T * H * 2 + T * H * 4
    layer_flops = 2.0 * n_slots * 3 * F * H
    res = {
        "workload": name, "T": T, "dtype": dt, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "layer_TBps": layer_bytes / (ms * 1e-3) / 1e12,
        "layer_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
        "layer_frac_of_mfma_peak": layer_flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[dt],
        "distinct_experts": distinct,
        "stages_ms": stages_ms,
        "route_only_ms": route_ms,
        "gate_up": {"ms": gu_ms, "bytes": gu_bytes, "flops": gu_flops,
                    "GBps": gu_bytes / (gu_ms * 1e-3) / 1e9,
                    "TFLOPs": gu_flops / (gu_ms * 1e-3) / 1e12},
        "bound": "hbm" if flop_per_byte < ridge else "mfma",
        "small_blocks": T * K <= 4 * sh.n_experts,
    }
    if routed:
        res["routed"] = {"workload": base, "expert_begin": routed[1], "expert_end": routed[2],
                         "local_slots": n_slots}
    del ws, out
    return res, d, ids


def measure_dense(bm, synthgen, torch, T, steps, warmup):
    """Beam's dense SwiGLU layer (hidden 5120, d_ff 20480, bf16) at T tokens: beam_dense_mlp_forward
    per step. MFMA-bound at prefill sizes: FLOP = 2 * T * 3 * hidden * d_ff."""
    d = synthgen.make_dense(T, device="cuda")
    H, F = d["hidden"], d["d_ff"]
    ws = torch.empty(bm.dense_workspace_bytes(H, F, bm.BEAM_BF16, T), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        bm.dense_mlp(d["x"], d["w_gate_up"], d["w_down"], out=out, workspace=ws, stream=stream)

    ms, gu_ms, stages_ms = timed_steps(bm, torch, step, steps, warmup, "gate_up")
    flops = 2.0 * T * 3 * H * F
    gu_flops = 2.0 * T * 2 * F * H
    res = {"workload": f"dense_prefill: Beam dense SwiGLU layer, T={T}, hidden {H}, d_ff {F}, bf16",
           "T": T, "dtype": "bf16", "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
           "layer_TFLOPs": flops / (ms * 1e-3) / 1e12,
           "layer_frac_of_mfma_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
           "stages_ms": stages_ms,
           "roofline": {"bound": "mfma", "kernel": "gate_up: grouped_pipe_kernel<true, false>",
                        "achieved": gu_flops / (gu_ms * 1e-3) / 1e12,
                        "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                        "frac": gu_flops / (gu_ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                        "traffic": None}}
    del ws, out, d
    return res


def measure_boundary(bm, synthgen, torch, weights, steps, warmup):
    """The post-MoE boundary at the prefill batch (T=8192): beam_moe_forward_boundary per step (the
    combine fused into output norm -> depth-scaled residual -> next norm), and the standalone
    beam_residual_boundary on an FP32 sublayer output. Both HBM-bound; algorithmic bytes per token:
    fused stage K*H*4 (Y slots) + H*2 (h) + 2*H*2 (h', x'); standalone H*4 + H*2 + 2*H*2."""
    wl = synthgen.WORKLOADS["prefill"]
    W = weights.get("bf16")
    d = synthgen.make_inputs(wl, device="cuda", with_experts=False)
    T, H, K = wl.T, wl.shape.hidden, wl.shape.topk
    cfg = bm.WorkloadCfg.of(wl.shape, "bf16", "bf16")
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    h = synthgen.normal((T, H), 1.0, 1, synthgen.TENSOR_IDS["residual"], "cuda", torch.bfloat16)
    gp = torch.ones(H, device="cuda")
    gn = torch.ones(H, device="cuda")
    h_out, x_next = torch.empty_like(h), torch.empty_like(h)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(fn, n):   # the boundary kernel is the library's combine stage
        ms, stage_ms, _ = timed_steps(bm, torch, fn, n, warmup, "combine")
        return ms, stage_ms

    fused_ms, fused_stage = run(lambda: bm.forward_boundary(
        d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg, h, gp, gn, 12, 1e-6,
        h_out=h_out, x_next=x_next, workspace=ws, stream=stream), steps)
    bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg, out=y,
               workspace=ws, stream=stream)
    _, alone = run(lambda: bm.residual_boundary(y, h, gp, gn, 12, 1e-6, h_out=h_out,
                                                x_next=x_next, stream=stream), 4 * steps)
    fused_bytes = T * (K * H * 4 + H * 2 + 2 * H * 2)
    alone_bytes = T * (H * 4 + H * 2 + 2 * H * 2)
    del ws, y
    return {"workload": "boundary_prefill: post-MoE boundary at T=8192 (hidden 5120, top-8)",
            "T": T, "ms_per_step": fused_ms, "tokens_per_s": T / (fused_ms * 1e-3),
            "fused_stage_ms": fused_stage, "standalone_ms": alone,
            "roofline": {"bound": "hbm", "kernel": "boundary_kernel<true> (combine fused)",
                         "achieved": fused_bytes / (fused_stage * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": fused_bytes / (fused_stage * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": None},
            "standalone_roofline": {"bound": "hbm", "kernel": "boundary_kernel<false>",
                                    "achieved": alone_bytes / (alone * 1e-3) / 1e9,
                                    "frac": alone_bytes / (alone * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def ceilings(torch):
    """Measured ceilings on this GPU, context for the roofline fractions (vendor library calls, not
    the measured path): HBM bandwidth of a 4 GiB device copy (read + write bytes); bf16 dense GEMM
    rate of an 8192^3 matmul; and a batched bf16 GEMM of the prefill gate/up shape (256 experts x
    256 rows x 5120 x 5120, dense, both operands contiguous)."""
    def clock(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    res = {}
    src = torch.empty(2 ** 30, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    t = clock(lambda: dst.copy_(src), 10)
    res["hbm_copy_GBps"] = 2 * src.numel() * 4 / t / 1e9
    del src, dst
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    t = clock(lambda: torch.mm(a, b), 10)
    res["bf16_gemm_8192_TFLOPs"] = 2.0 * 8192 ** 3 / t / 1e12
    del a, b
    w = (torch.randn(256, 5120, 5120, device="cuda") * 0.02).to(torch.bfloat16)
    xt = torch.randn(256, 5120, 256, device="cuda").to(torch.bfloat16)
    o = torch.empty(256, 5120, 256, device="cuda", dtype=torch.bfloat16)
    t = clock(lambda: torch.bmm(w, xt, out=o), 5)
    res["bf16_batched_gemm_gate_up_shape_TFLOPs"] = 2.0 * 256 * 256 * 5120 * 5120 / t / 1e12
    del w, xt, o
    torch.cuda.empty_cache()
    res["note"] = ("vendor-library rates on this GPU for context; the bench's kernels are the "
                   "library's own HIP kernels")
    return res


def roofline(r, workload):
    g = r["gate_up"]
    if r["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": g["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": g["GBps"] / HBM_PEAK_GBS}
    else:
        pk = PEAK_TFLOPS[r["dtype"]]
        roof = {"bound": "mfma", "achieved": g["TFLOPs"], "peak": pk, "unit": "TFLOP/s",
                "frac": g["TFLOPs"] / pk}
    fp8 = str(r["dtype"] == "fp8").lower()
    if r["small_blocks"]:   # K split over 4 waves
        roof["kernel"] = f"gate_up: grouped_small_ks_kernel<true, {fp8}, 4>"
    else:
        roof["kernel"] = f"gate_up: grouped_pipe_kernel<true, {fp8}>"
    roof["algorithmic_bytes_per_launch"] = g["bytes"]
    roof["traffic"] = None
    cpath = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if os.path.exists(cpath):
        with open(cpath) as f:
            c = json.load(f)
        if c.get("kernel_source_hash") == kernel_source_hash():
            roof["traffic"] = c.get("gate_up_hbm_bytes_per_launch")
    return roof


def cpu_baseline(torch, synthgen, d, W, wl_name, n_tok):
    """The oracle as it stands, on the host cores: full-batch routing plus the expert MLPs and
    combine of the first n_tok tokens (their experts' weights copied to the host beforehand)."""
    from oracle import experts, router
    wl = synthgen.WORKLOADS[wl_name]
    sh = wl.shape
    x_h, wr_h, b_h = d["x"].cpu(), W["w_router"].cpu(), d["bias"].cpu()
    toks = list(range(n_tok))
    r0 = router.route(x_h[:n_tok], wr_h, b_h, sh.n_groups, sh.topk_groups, sh.topk,
                      sh.routed_scale)
    need = sorted(set(int(e) for e in r0.ids.ravel()))
    host_w = {e: (W["w_gate_up"][e].cpu(), W["w_down"][e].cpu()) for e in need}
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    t0 = time.perf_counter()
    r = router.route(x_h, wr_h, b_h, sh.n_groups, sh.topk_groups, sh.topk, sh.routed_scale)
    t_route = time.perf_counter() - t0
    get = lambda e: experts.split_expert(host_w[e][0], host_w[e][1], sh.d_ff)  # noqa: E731
    t1 = time.perf_counter()
    experts.forward_expert_major(x_h[:n_tok], r.ids[toks], r.weights[toks], get, "bf16")
    t_exp = time.perf_counter() - t1
    # per-token cost of the whole block: routing amortised over the batch + experts per token
    per_tok = t_route / wl.T + t_exp / n_tok
    res = {"value": 1.0 / per_tok, "unit": "tokens/s",
           "cores": int(max(blas, torch.get_num_threads())), "kind": "oracle",
           "sample": f"{wl_name}: routing of all {wl.T} tokens ({t_route:.2f} s) + expert MLPs and "
                     f"combine of {n_tok} tokens / {n_tok * sh.topk} expert calls ({t_exp:.2f} s), "
                     f"float64 numpy"}
    # the same on one core, on a smaller sample (routing of all tokens, experts of n1 tokens)
    try:
        from threadpoolctl import threadpool_limits
        n1 = max(1, n_tok // 8)
        nt = torch.get_num_threads()
        torch.set_num_threads(1)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            r1 = router.route(x_h, wr_h, b_h, sh.n_groups, sh.topk_groups, sh.topk,
                              sh.routed_scale)
            t_route1 = time.perf_counter() - t0
            t1 = time.perf_counter()
            experts.forward_expert_major(x_h[:n1], r1.ids[:n1], r1.weights[:n1], get, "bf16")
            t_exp1 = time.perf_counter() - t1
        torch.set_num_threads(nt)
        res["one_core"] = {"value": 1.0 / (t_route1 / wl.T + t_exp1 / n1), "unit": "tokens/s",
                           "sample": f"routing of all {wl.T} tokens ({t_route1:.2f} s) + experts "
                                     f"of {n1} tokens ({t_exp1:.2f} s), 1 thread"}
    except ImportError:
        res["one_core"] = None
    return res


def measure_small_t(bm, synthgen, torch, weights, steps, warmup, Ts=(1, 2, 4, 8, 16, 64)):
    """The decode-shaped layer at small token counts: ms per step (wall clock over `steps` calls,
    no timing events), distinct experts touched, and the HBM floor of the weights they stream."""
    wl = synthgen.WORKLOADS["decode"]
    W = weights.get("bf16")
    sh = wl.shape
    cfg = bm.WorkloadCfg.of(sh, wl.x_dtype, wl.w_dtype)
    stream = torch.cuda.current_stream()
    per_expert = 3 * sh.d_ff * sh.hidden * 2   # gate, up and down rows, bf16
    res = {}
    for T in Ts:
        d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False)
        ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
        out = torch.empty((T, sh.hidden), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, sh.topk), dtype=torch.int32, device="cuda")

        def step():
            bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg,
                       out=out, topk_ids_out=ids, workspace=ws, stream=stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        distinct = int(torch.unique(ids).numel())
        floor = distinct * per_expert / (HBM_PEAK_GBS * 1e9) * 1e3
        res[str(T)] = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                       "distinct_experts": distinct, "hbm_floor_ms": floor,
                       "frac_of_floor": floor / ms}
    return res


def summarize_counters(workload: str, fetch_dir: str, write_dir: str) -> None:
    """Writes profiles/counters_<workload>.{json,txt} from two rocprofv3 --pmc runs of this script
    (FETCH_SIZE, then WRITE_SIZE, each with --copy-probe-gib 1): per-kernel KiB per dispatch averaged
    over the run's dispatches, scaled to bytes by what the same counter reads for the 1 GiB device
    copy (read once, written once)."""
    import csv
    import collections

    def dispatches(d, counter):
        vals = collections.defaultdict(list)
        for root, _, files in os.walk(d):
            for fn in files:
                if fn.endswith("counter_collection.csv"):
                    with open(os.path.join(root, fn)) as f:
                        for r in csv.DictReader(f):
                            if r["Counter_Name"] == counter:
                                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fd, wd = dispatches(fetch_dir, "FETCH_SIZE"), dispatches(write_dir, "WRITE_SIZE")
    fetch = {k: sum(v) / len(v) for k, v in fd.items()}
    write = {k: sum(v) / len(v) for k, v in wd.items()}
    # the probe is the largest copy dispatch (smaller copies of the run share its kernel)
    copy = [k for k in fd if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no copy-probe dispatch in the FETCH_SIZE run (--copy-probe-gib 1)")
    probe = 2 ** 30
    f_copy = max(max(fd[k]) for k in copy)
    w_copy = max(max(wd.get(k, [0.0])) for k in copy)
    fs, ws = probe / (1024 * f_copy), probe / (1024 * w_copy)
    short = {}
    for k in fetch:
        if "beam::" in k:
            name = k.split("(")[0].replace("void ", "")
            short[name] = {"FETCH_SIZE_KiB": fetch[k], "WRITE_SIZE_KiB": write.get(k, 0.0),
                           "hbm_bytes": 1024 * (fs * fetch[k] + ws * write.get(k, 0.0))}
    gu = [n for n in short if n.startswith("beam::grouped_") and "<true" in n]
    out = {"workload": workload, "kernel": gu[0] if gu else None,
           "kernel_source_hash": kernel_source_hash(), "fetch_scale": fs, "write_scale": ws,
           "copy_probe": {"bytes": probe, "FETCH_SIZE_KiB": f_copy, "WRITE_SIZE_KiB": w_copy},
           "gate_up_hbm_bytes_per_launch": short[gu[0]]["hbm_bytes"] if gu else None,
           "per_kernel": short}
    base = os.path.join(ROOT, "profiles", f"counters_{workload}")
    with open(base + ".json", "w") as f:
        json.dump(out, f, indent=1)
    cmd = ('rocprofv3 --pmc {c} --kernel-include-regex "beam::|copyBuffer" --output-format csv '
           '-d $R/gpurun_out/pmc_{w}_{c} -o run -- python $R/bench.py --workload {w} --also "" '
           '--steps 3 --warmup 1 --no-cpu-baseline --no-ceilings --copy-probe-gib 1')
    lines = [f"# HBM traffic per dispatch from rocprofv3 counters, workload {workload}", "",
             "commands (from /tmp with TMPDIR=/tmp, repository root $R; one pass per counter):",
             "  " + cmd.format(c="FETCH_SIZE", w=workload),
             "  " + cmd.format(c="WRITE_SIZE", w=workload),
             f"summary: python $R/bench.py --summarize-counters {workload} "
             f"$R/gpurun_out/pmc_{workload}_FETCH_SIZE $R/gpurun_out/pmc_{workload}_WRITE_SIZE", "",
             f"copy probe (device copy of 1 GiB = 1048576 KiB): FETCH_SIZE {f_copy:.1f} KiB, "
             f"WRITE_SIZE {w_copy:.1f} KiB", f"-> scale factors: FETCH x{fs:.4f}, WRITE x{ws:.4f}",
             "", f"{'kernel':<55}{'FETCH_KiB':>13}{'WRITE_KiB':>13}{'HBM_bytes(scaled)':>19}"]
    for n, v in short.items():
        lines.append(f"{n[:54]:<55}{v['FETCH_SIZE_KiB']:>13.1f}{v['WRITE_SIZE_KiB']:>13.1f}"
                     f"{v['hbm_bytes']:>19.4g}")
    with open(base + ".txt", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {base}.json / .txt")


def summarize_trace(trace_dir: str, which: str = "all") -> None:
    """Writes profiles/kernels_bench_all_workloads.txt (which = "all": a default bench.py run) or
    profiles/kernels_bench_decode.txt (which = "decode": bench.py --also "", the headline decode leg
    alone, so its gate/up kernel's average can be set beside the bench line's) from the
    kernel_stats.csv of `rocprofv3 --kernel-trace --stats --output-format csv`: the library's
    kernels with their call counts and average / min / max durations."""
    import csv
    rows = []
    for root, _, files in os.walk(trace_dir):
        for fn in files:
            if fn.endswith("kernel_stats.csv"):
                with open(os.path.join(root, fn)) as f:
                    rows += [r for r in csv.DictReader(f) if "beam::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if which == "decode":
        head = ["# rocprofv3 kernel-trace stats: bench.py headline leg only (decode T=32: 5 warm-up",
                "# + 50 timed steps, 50 instrumented, 50 with an event pair per step, route-only calls)",
                "", "command (from /tmp with TMPDIR=/tmp, repository root $R):",
                "  rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_decode "
                "-o dec -- python $R/bench.py --also \"\" --no-cpu-baseline --no-ceilings",
                "summary: python $R/bench.py --summarize-trace $R/gpurun_out/prof_decode decode", ""]
    else:
        head = [
            "# rocprofv3 kernel-trace stats: bench.py default run (decode T=32 headline; legs",
            "# prefill T=8192, skew T=32768, fp8_decode T=32, fp8_prefill T=8192, routed_prefill",
            "# (experts 32..63 of the T=8192 batch), dense_prefill (dense SwiGLU d_ff 20480,",
            "# T=8192), boundary_prefill (post-MoE boundary, T=8192), small_t (T = 1 .. 64))", "",
            "command (from /tmp with TMPDIR=/tmp, repository root $R):",
            "  rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_all -o all "
            "-- python $R/bench.py",
            "summary: python $R/bench.py --summarize-trace $R/gpurun_out/prof_all", ""]
    lines = head + [
        "Template arguments: grouped_*<GATE_UP, FP8, ...>: <true,*> gate/up, <false,*> down;",
        "small_ks = 16-row blocks, K split across 8 or 4 waves (decode legs); pipe = 320-row blocks",
        "(prefill legs). router_fused_kernel (with router_split_kernel before it): the one-pass router",
        "past 1024 tokens; router_partial_kernel + select: up to 1024 tokens.", "",
        f"{'kernel':<62}{'calls':>8}{'avg_us':>11}{'min_us':>11}{'max_us':>11}"]
    for r in rows:
        name = r["Name"].replace("void ", "").split("(")[0]
        lines.append(f"{name[:61]:<62}{int(r['Calls']):>8}{float(r['AverageNs']) / 1e3:>11.1f}"
                     f"{float(r['MinNs']) / 1e3:>11.1f}{float(r['MaxNs']) / 1e3:>11.1f}")
    out = os.path.join(ROOT, "profiles", "kernels_bench_decode.txt" if which == "decode"
                       else "kernels_bench_all_workloads.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        summarize_counters(*sys.argv[2:5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        summarize_trace(*sys.argv[2:4])
        return
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the library has no "
              "multi-GPU path. Across GPUs the block would shard by experts (one group of 32 per "
              "GPU, an all-to-all dispatch and combine around beam_moe_forward_routed).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import routing_grouped_expert_fp32_amd as bm
    import synthgen
    bm.lib()
    torch.cuda.set_device(0)
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    weights = Weights(synthgen, torch)
    main_res, d, ids = measure(bm, synthgen, torch, a.workload, weights, a.steps, a.warmup)
    print(f"[bench] {a.workload}: {main_res['ms_per_step']:.3f} ms/step", file=sys.stderr,
          flush=True)
    extra = {}
    for name in [s for s in a.also.split(",") if s and s != a.workload]:
        if name == "boundary_prefill":
            r = measure_boundary(bm, synthgen, torch, weights, max(5, a.steps // 5), a.warmup)
            extra[name] = r
            print(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
            continue
        if name == "small_t":
            r = measure_small_t(bm, synthgen, torch, weights, max(10, a.steps // 2), a.warmup)
            extra[name] = r
            print(f"[bench] {name}: " + ", ".join(f"T={t} {v['ms_per_step']:.3f} ms"
                                                 for t, v in r.items()), file=sys.stderr, flush=True)
            continue
        if name == "dense_prefill":
            r = measure_dense(bm, synthgen, torch, 8192, max(5, a.steps // 5), a.warmup)
            extra[name] = r
            print(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
            continue
        r, _, _ = measure(bm, synthgen, torch, name, weights, max(5, a.steps // 2), a.warmup)
        r["roofline"] = roofline(r, name)
        extra[name] = r
        print(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    if a.copy_probe_gib > 0:
        n = int(a.copy_probe_gib * 2 ** 30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceil = None
    if not a.no_ceilings:
        print("[bench] measuring HBM and GEMM ceilings", file=sys.stderr, flush=True)
        ceil = ceilings(torch)
    cpu = None
    wl = synthgen.WORKLOADS[ROUTED.get(a.workload, (a.workload,))[0]]
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(torch, synthgen, d, weights.get(wl.w_dtype),
                           ROUTED.get(a.workload, (a.workload,))[0], a.cpu_tokens)
    sh = wl.shape
    line = {
        "metric": "MoE-layer tokens/sec (d5120, 256 exp, top-8) at T=32 and T=8192; % of roofline",
        "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": main_res["dtype"], "data": "synthetic",
        "config": {"workload": f"{a.workload}: Beam MoE layer, T={wl.T}, hidden {sh.hidden}, "
                               f"{sh.n_experts} experts ({sh.n_groups} groups, keep "
                               f"{sh.topk_groups}), top-{sh.topk}, d_ff {sh.d_ff}, "
                               f"{main_res['dtype']} experts, FP32 router, fp32 out",
                   "T": wl.T, "global_batch": wl.T, "parallelism": "single GPU"},
        "roofline": roofline(main_res, a.workload),
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "detail": main_res,
        "also": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
