"""GPU parity of beam_dense_mlp_forward (a dense SwiGLU layer run as one expert with weight 1;
Beam's dense layers: [V] §MoE and residual stream, [H] §专家混合), through the C ABI, against the
oracle's expert MLP under the same bf16 / FP8 contracts."""
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


def _run(d, w_dtype, out_dtype=bm.BEAM_F32):
    kw = {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=d["w_gate_up_scale"], w_down_scale=d["w_down_scale"])
    out = bm.dense_mlp(d["x"], d["w_gate_up"], d["w_down"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out


def _oracle(d, w_dtype, toks):
    ex = experts.split_expert(d["w_gate_up"].cpu(), d["w_down"].cpu(), d["d_ff"],
                              d["w_gate_up_scale"].cpu() if w_dtype == "fp8" else None,
                              d["w_down_scale"].cpu() if w_dtype == "fp8" else None)
    xr = d["x"][torch.from_numpy(toks).to(d["x"].device)].cpu()
    return experts.expert_mlp(xr, ex, w_dtype)


@pytest.mark.parametrize("w_dtype,T,d_ff", [("bf16", 3, 1024), ("bf16", 100, 1024),
                                            ("bf16", 600, 1024), ("fp8", 5, 1024),
                                            ("fp8", 600, 1024), ("bf16", 600, 4096),
                                            ("bf16", 1000, 4096)])
def test_small_dense_all_tokens(w_dtype, T, d_ff):
    """hidden 512: decode-sized (16-row blocks) and tiled paths; with d_ff 4096 the few tiled
    workgroups make the bf16 down GEMM split K into 4 parts of 16 stages (FP8 splits are covered
    at Beam's dense shape below)."""
    _say("dense small", w_dtype, T, d_ff)
    d = synthgen.make_dense(T, 512, d_ff, w_dtype, device="cuda", sigma_w=0.05)
    out = _run(d, w_dtype).cpu().numpy()
    ref = _oracle(d, w_dtype, np.arange(T))
    err, rms = parity.rel_err(out, ref)
    p999 = float(np.quantile(np.abs(out - ref), 0.999) / rms)
    _say("dense small", w_dtype, T, "max|err|/rms", err, "p99.9", p999)
    if w_dtype == "fp8" and T * d["hidden"] > 64 * 512:
        # Over many elements the FP8 bar meets its boundary flips: where the FP32 and FP64 paths
        # put h (or its row amax) on different sides of a bf16 / E4M3 rounding boundary, an E4M3
        # code moves by one step (6-12 %). Such flips are rare (median error ~5e-5) but their
        # largest effect over ~3e5 outputs reaches ~5e-2; the tail is checked at the 99.9th
        # percentile and the maximum at twice the bar.
        assert p999 <= parity.FP8_P999 and err <= 2 * parity.TOL["fp8"]
    else:
        assert err <= parity.TOL[w_dtype]


@pytest.fixture(scope="module")
def beam_dense():
    _say("generating Beam dense layer (5120 x 20480, bf16) on cuda:0")
    d = synthgen.make_dense(8192, device="cuda")
    torch.cuda.synchronize()
    return d


def test_beam_dense_prefill_sampled(beam_dense):
    """Beam's dense layer at T = 8192, in the launch configuration the benchmark times; sampled
    tokens against the oracle, and the bf16 output is the rounded FP32 output."""
    out = _run(beam_dense, "bf16")
    toks = np.array([0, 1, 777, 4095, 6000, 8191])
    ref = _oracle(beam_dense, "bf16", toks)
    err, rms = parity.rel_err(out[torch.from_numpy(toks).cuda()].cpu().numpy(), ref)
    _say("Beam dense T=8192 sampled max|err|/rms", err)
    assert err <= parity.TOL["bf16"]
    out16 = _run(beam_dense, "bf16", bm.BEAM_BF16)
    assert torch.equal(out16, out.to(torch.bfloat16))


def test_beam_dense_decode_all_tokens(beam_dense):
    d = dict(beam_dense)
    d["x"] = beam_dense["x"][:32].contiguous()
    d["T"] = 32
    out = _run(d, "bf16").cpu().numpy()
    ref = _oracle(d, "bf16", np.arange(32))
    err, rms = parity.rel_err(out, ref)
    _say("Beam dense T=32 max|err|/rms", err)
    assert err <= parity.TOL["bf16"]


def test_beam_dense_fp8_sampled():
    """Beam's dense layer with FP8 weights at T = 8192 (the down GEMM splits K into 4 parts),
    sampled tokens against the oracle's FP8 contract; and at T = 32 every token."""
    _say("generating Beam dense layer (5120 x 20480, FP8) on cuda:0")
    d = synthgen.make_dense(8192, w_dtype="fp8", device="cuda")
    torch.cuda.synchronize()
    out = _run(d, "fp8")
    toks = np.array([0, 1, 777, 4095, 6000, 8191])
    ref = _oracle(d, "fp8", toks)
    err, rms = parity.rel_err(out[torch.from_numpy(toks).cuda()].cpu().numpy(), ref)
    _say("Beam dense FP8 T=8192 sampled max|err|/rms", err)
    assert err <= parity.TOL["fp8"]
    d32 = dict(d)
    d32["x"] = d["x"][:32].contiguous()
    d32["T"] = 32
    out = _run(d32, "fp8").cpu().numpy()
    err, rms = parity.rel_err(out, _oracle(d32, "fp8", np.arange(32)))
    _say("Beam dense FP8 T=32 max|err|/rms", err)
    assert err <= parity.TOL["fp8"]
