"""GPU parity of the sublayer boundary (output RMSNorm -> depth-scaled residual -> next RMSNorm,
[V] §MoE and residual stream, §Agent-driven optimization items 1 and 3; [S] §Sandwich Normalization
and Depth-Scaled Residuals) through the C ABI, standalone and fused with the MoE combine.

The outputs are bf16, so they are compared in bf16 units in the last place (taken at the larger of
the value and its row's rms, see ulp_stats): where the FP32 kernel and the FP64 oracle put a value on
different sides of a bf16 rounding boundary they differ by one ulp, and such a step can carry through
the later roundings of the chain (p -> b -> h' -> x'). The bar: every element within 2 ulps, and at
least 99% of them equal (MoE-fused: 95%, since y itself then differs between the FP32 and FP64
expert paths by ~1e-4 relative)."""
import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import boundary, experts, router

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _say(*a):
    print(*a, flush=True)


def ulp_stats(gpu, ref):
    """(max distance, fraction equal) in bf16 ulps, the ulp taken at max(|ref|, rms of the row):
    a value near zero from a cancelling add (a + b with a ~ -b) inherits the ulps of its operands,
    which are ~ the row's scale, not the tiny ulp of the result."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    scale = np.maximum(np.abs(ref), rms)
    ulp = np.exp2(np.floor(np.log2(scale)) - 7)
    d = np.abs(gpu - ref) / ulp
    return float(d.max()), float((gpu == ref).mean())


def _inputs(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn((T, H), generator=g) * 3.0
    h = torch.randn((T, H), generator=g).to(torch.bfloat16)
    gp = 1.0 + (torch.rand(H, generator=g) - 0.5) * 0.4
    gn = 1.0 + (torch.rand(H, generator=g) - 0.5) * 0.4
    return y, h, gp, gn


@pytest.mark.parametrize("T,H,ydt,n", [(37, 5120, "f32", 7), (37, 5120, "bf16", 7),
                                       (5, 512, "f32", 2), (3, 768, "f32", 100),
                                       (2, 16384, "f32", 1), (300, 5120, "f32", 55)])
def test_boundary_against_oracle(T, H, ydt, n):
    _say("boundary", T, H, ydt, n)
    y, h, gp, gn = _inputs(T, H, T * 1000 + H)
    if ydt == "bf16":
        y = y.to(torch.bfloat16)
    h_out, x_next = bm.residual_boundary(y.cuda(), h.cuda(), gp.cuda(), gn.cuda(), n, EPS)
    torch.cuda.synchronize()
    rh, rx = boundary.boundary(y.float().numpy(), h.float().numpy(), gp.numpy(), gn.numpy(), n,
                               EPS)
    mh, eh = ulp_stats(h_out.float().cpu().numpy(), rh)
    mx, ex = ulp_stats(x_next.float().cpu().numpy(), rx)
    _say(f"h': max {mh} ulp, {eh:.5f} equal; x': max {mx} ulp, {ex:.5f} equal")
    assert mh <= 2 and mx <= 2 and eh >= 0.99 and ex >= 0.99


def test_boundary_in_place_equals_out_of_place():
    y, h, gp, gn = _inputs(17, 5120, 3)
    y, h, gp, gn = y.cuda(), h.cuda(), gp.cuda(), gn.cuda()
    h_out, x_next = bm.residual_boundary(y, h, gp, gn, 9, EPS)
    h2 = h.clone()
    h2_out, x2 = bm.residual_boundary(y, h2, gp, gn, 9, EPS, h_out=h2)
    torch.cuda.synchronize()
    assert h2_out.data_ptr() == h2.data_ptr()
    assert torch.equal(h2, h_out) and torch.equal(x2, x_next)


@pytest.fixture(scope="module")
def beam_bf16():
    _say("generating Beam bf16 weights on cuda:0")
    d = synthgen.make_inputs("prefill", device="cuda", T=1)
    torch.cuda.synchronize()
    return d


def _moe(name, W, T=None):
    wl = synthgen.WORKLOADS[name]
    d = synthgen.make_inputs(wl, device="cuda", T=T, with_experts=False)
    cfg = bm.WorkloadCfg.of(wl.shape, "bf16", "bf16")
    return wl, d, cfg


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fused_equals_forward_then_boundary(beam_bf16, name):
    """The MoE-fused boundary sums the slots in the combine's order: bitwise equal to the standalone
    boundary applied to beam_moe_forward's FP32 output."""
    wl, d, cfg = _moe(name, beam_bf16)
    T = d["T"]
    _, h, gp, gn = _inputs(T, 5120, 11)
    h, gp, gn = h.cuda(), gp.cuda(), gn.cuda()
    W = beam_bf16
    out = bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg)
    rh, rx = bm.residual_boundary(out, h, gp, gn, 12, EPS)
    fh, fx = bm.forward_boundary(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"],
                                 cfg, h, gp, gn, 12, EPS)
    torch.cuda.synchronize()
    assert torch.equal(fh, rh) and torch.equal(fx, rx)


def test_fused_decode_against_oracle(beam_bf16):
    wl, d, cfg = _moe("decode", beam_bf16)
    T = d["T"]
    _, h, gp, gn = _inputs(T, 5120, 12)
    W = beam_bf16
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    fh, fx = bm.forward_boundary(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"],
                                 cfg, h.cuda(), gp.cuda(), gn.cuda(), 12, EPS, topk_ids_out=ids)
    torch.cuda.synchronize()
    sh = wl.shape
    r = router.route(d["x"].cpu(), W["w_router"].cpu(), d["bias"].cpu(), sh.n_groups,
                     sh.topk_groups, sh.topk, sh.routed_scale)
    ids_c = ids.cpu().numpy()
    assert not parity.check_routing(ids_c, router.weights(r.s, ids_c.astype(np.int64), 2.5),
                                    r)["failures"]
    get = parity.expert_loader(W["w_gate_up"], W["w_down"], sh.d_ff)
    y = experts.forward_expert_major(router.to_f64(d["x"].cpu()), r.ids, r.weights, get, "bf16")
    rh, rx = boundary.boundary(y, h.float().numpy(), gp.numpy(), gn.numpy(), 12, EPS)
    mh, eh = ulp_stats(fh.float().cpu().numpy(), rh)
    mx, ex = ulp_stats(fx.float().cpu().numpy(), rx)
    _say(f"fused decode: h' max {mh} ulp, {eh:.5f} equal; x' max {mx} ulp, {ex:.5f} equal")
    assert mh <= 2 and mx <= 2 and eh >= 0.95 and ex >= 0.95
