"""GPU parity of beam_moe_forward_routed: the expert steps from given routes over a range of experts
(routing replay, [S] §Reinforcement learning in Miles; the expert-parallel entry point, [S] §Fusion
Optimizations), through the C ABI, against the CPU oracle and against beam_moe_forward.
"""
import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import experts

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def beam_bf16():
    _say("generating Beam bf16 weights on cuda:0")
    d = synthgen.make_inputs("prefill", device="cuda", T=1)
    torch.cuda.synchronize()
    return d


def _cfg(wl, out="f32"):
    return bm.WorkloadCfg.of(wl.shape, wl.x_dtype, wl.w_dtype, out)


def _forward(name, weights, T=None):
    wl = synthgen.WORKLOADS[name]
    d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False)
    T = d["T"]
    ids = torch.empty((T, wl.shape.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.shape.topk), dtype=torch.float32, device="cuda")
    out = bm.forward(d["x"], weights["w_router"], d["bias"], weights["w_gate_up"],
                     weights["w_down"], _cfg(wl), topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    return wl, d, out, ids, w


def _routed(wl, x, ids, w, weights, b, e, **kw):
    out = bm.forward_routed(x, ids, w, weights["w_gate_up"][b:e], weights["w_down"][b:e], _cfg(wl),
                            b, e, **kw)
    torch.cuda.synchronize()
    return out


def _rel(a, b):
    a = a.double()
    b = b.double()
    return float((a - b).abs().max() / b.pow(2).mean().sqrt())


@pytest.mark.parametrize("name,T", [("decode", None), ("decode", 300), ("prefill", None)])
def test_full_range_equals_forward(beam_bf16, name, T):
    wl, d, out, ids, w = _forward(name, beam_bf16, T)
    _say("routed full range", name, d["T"])
    got = _routed(wl, d["x"], ids, w, beam_bf16, 0, wl.shape.n_experts)
    assert bool((got == out).all())   # same kernels, same order (the sum starts from +0)


@pytest.mark.parametrize("name,T", [("decode", None), ("prefill", None)])
def test_expert_parallel_partition_sums_to_forward(beam_bf16, name, T):
    """Eight ranks of one group (32 experts) each: their partial outputs add up to the layer."""
    wl, d, out, ids, w = _forward(name, beam_bf16, T)
    _say("routed EP8 partition", name, d["T"])
    total = torch.zeros_like(out)
    for r in range(8):
        total += _routed(wl, d["x"], ids, w, beam_bf16, 32 * r, 32 * (r + 1))
    err = _rel(total, out)
    _say("partition vs forward max|err|/rms", err)
    assert err <= 1e-5


def test_given_routes_against_oracle(beam_bf16):
    """Arbitrary routes (not the router's), weights used as given, ids outside the range or outside
    [0, E) skipped; the local weights hold experts [64, 160) only."""
    wl = synthgen.WORKLOADS["decode"]
    T, K, E = 40, wl.shape.topk, wl.shape.n_experts
    d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    ids[3, 2] = -1
    ids[7, 5] = 999
    ids[11, :] = rng.choice(np.arange(0, 64), size=K, replace=False)   # no local expert: zeros
    w = rng.uniform(-0.5, 1.5, size=(T, K)).astype(np.float32)
    b, e = 64, 160
    got = _routed(wl, d["x"], torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), beam_bf16,
                  b, e).cpu()
    assert bool((got[11] == 0).all())
    get = parity.expert_loader(beam_bf16["w_gate_up"], beam_bf16["w_down"], wl.shape.d_ff)
    ref = experts.forward_routed(d["x"].cpu(), ids, w, get, "bf16", b, e)
    err, rms = parity.rel_err(got.numpy(), ref)
    _say("given routes bf16 max|err|/rms", err)
    assert err <= parity.TOL["bf16"]


def test_prefill_expert_share_sampled(beam_bf16):
    """One expert-parallel share (experts 32..63) at the prefill batch, tiled GEMM path, sampled
    tokens against the oracle."""
    wl, d, out, ids, w = _forward("prefill", beam_bf16)
    b, e = 32, 64
    got = _routed(wl, d["x"], ids, w, beam_bf16, b, e).cpu().numpy()
    ids_c, w_c = ids.cpu().numpy(), w.cpu().numpy()
    local = np.nonzero(((ids_c >= b) & (ids_c < e)).any(axis=1))[0]
    toks = np.sort(np.random.default_rng(3).choice(local, size=10, replace=False))
    get = parity.expert_loader(beam_bf16["w_gate_up"], beam_bf16["w_down"], wl.shape.d_ff)
    ref = experts.forward_routed(d["x"][torch.from_numpy(toks).cuda()].cpu(), ids_c[toks],
                                 w_c[toks], get, "bf16", b, e)
    err, rms = parity.rel_err(got[toks], ref)
    _say("prefill share sampled max|err|/rms", err)
    assert err <= parity.TOL["bf16"]
    assert np.all(got[np.setdiff1d(np.arange(d["T"]), local)] == 0)


def test_empty_range_and_zero_tokens(beam_bf16):
    wl, d, out, ids, w = _forward("decode", beam_bf16)
    got = _routed(wl, d["x"], ids, w, beam_bf16, 17, 17)
    assert bool((got == 0).all())
    x0 = d["x"][:0]
    empty = bm.forward_routed(x0, ids[:0], w[:0], beam_bf16["w_gate_up"], beam_bf16["w_down"],
                              _cfg(wl), 0, 256)
    assert empty.shape[0] == 0


def test_tiny_fp32_range_all_tokens():
    wl = synthgen.WORKLOADS["tiny"]
    d = synthgen.make_inputs(wl, device="cuda")
    T, K = d["T"], wl.shape.topk
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], _cfg(wl),
               topk_ids_out=ids, topk_w_out=w)
    b, e = 4, 20
    got = _routed(wl, d["x"], ids, w, d, b, e).cpu().numpy()
    get = parity.expert_loader(d["w_gate_up"], d["w_down"], wl.shape.d_ff)
    ref = experts.forward_routed(d["x"].cpu(), ids.cpu().numpy(), w.cpu().numpy(), get, "fp32",
                                 b, e)
    err, rms = parity.rel_err(got, ref)
    _say("tiny fp32 range max|err|/rms", err)
    assert err <= parity.TOL["f32"]


def test_fp8_decode_range():
    wl = synthgen.WORKLOADS["fp8_decode"]
    weights = synthgen.make_inputs("fp8_decode", device="cuda", T=1)
    d = synthgen.make_inputs(wl, device="cuda", with_experts=False)
    T, K = d["T"], wl.shape.topk
    cfg = bm.WorkloadCfg.of(wl.shape, "bf16", "fp8")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    bm.forward(d["x"], weights["w_router"], d["bias"], weights["w_gate_up"], weights["w_down"],
               cfg, w_gate_up_scale=weights["w_gate_up_scale"],
               w_down_scale=weights["w_down_scale"], topk_ids_out=ids, topk_w_out=w)
    b, e = 0, 96
    got = bm.forward_routed(d["x"], ids, w, weights["w_gate_up"][b:e], weights["w_down"][b:e],
                            cfg, b, e, w_gate_up_scale=weights["w_gate_up_scale"][b:e],
                            w_down_scale=weights["w_down_scale"][b:e])
    torch.cuda.synchronize()
    get = parity.expert_loader(weights["w_gate_up"], weights["w_down"], wl.shape.d_ff,
                               weights["w_gate_up_scale"], weights["w_down_scale"])
    ref = experts.forward_routed(d["x"].cpu(), ids.cpu().numpy(), w.cpu().numpy(), get, "fp8",
                                 b, e)
    err, rms = parity.rel_err(got.cpu().numpy(), ref)
    _say("fp8 decode range max|err|/rms", err)
    assert err <= parity.TOL["fp8"]


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_tiled_range_every_row(w_dtype):
    """A routed call over one group of experts (32..63) at T = 300 (tiled kernels; FP8 quantises only
    the call's own sorted rows) through the every-row check (fullcheck.py): each local row's h, codes
    and output, and every token's sum over its local slots at the bar except counted near-flip
    tokens."""
    import fullcheck
    name = "fp8_decode" if w_dtype == "fp8" else "decode"
    wl = synthgen.WORKLOADS[name]
    W = synthgen.make_inputs(name, device="cuda", T=1)
    d = synthgen.make_inputs(wl, device="cuda", T=300, with_experts=False)
    cfg = bm.WorkloadCfg.of(wl.shape, "bf16", w_dtype)
    T, b, e = 300, 32, 64
    kw, kw_l = {}, {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=W["w_gate_up_scale"], w_down_scale=W["w_down_scale"])
        kw_l = dict(w_gate_up_scale=W["w_gate_up_scale"][b:e], w_down_scale=W["w_down_scale"][b:e])
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg,
               topk_ids_out=ids, topk_w_out=w, **kw)
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out = bm.forward_routed(d["x"], ids, w, W["w_gate_up"][b:e], W["w_down"][b:e], cfg, b, e,
                            workspace=ws, **kw_l)
    torch.cuda.synchronize()
    ids_c = ids.cpu().numpy().astype(np.int64)
    local = np.where((ids_c >= b) & (ids_c < e), ids_c - b, -1)
    fp8 = w_dtype == "fp8"

    def get(i):
        return fullcheck.expert_f64(W["w_gate_up"][b + i], W["w_down"][b + i], wl.shape.d_ff,
                                    W["w_gate_up_scale"][b + i] if fp8 else None,
                                    W["w_down_scale"][b + i] if fp8 else None)
    st = fullcheck.read_state(ws, cfg, T, fp8)
    stats = fullcheck.check_batch(out, d["x"], local, w.cpu().numpy().astype(np.float64), st, get,
                                  w_dtype, e - b, say=_say, routed=True)
    assert stats["rows_checked"] == int((local >= 0).sum())
    assert stats["tokens_checked"] == int((local >= 0).any(axis=1).sum())
    assert stats["err_out_pure"] <= parity.TOL[w_dtype], stats
    assert stats["near_flip_tokens"] <= max(2, T // 50), stats
