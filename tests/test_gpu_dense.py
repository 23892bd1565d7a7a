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
    if w_dtype == "fp8":
        # one expert at a toy width: no combine averages the FP8 instructions' summation error over
        # experts, and the end-to-end bar is held at the layer's real width below
        # (test_beam_dense_fp8_every_token); every step is checked here against the GPU's own
        # intermediate values within their bounds
        stats, _ = _fp8_every_row(d, bar=False)
        _say("toy dense FP8: max|err|/rms against the exact-sum oracle", stats["err_out_pure"])
        return
    out = _run(d, w_dtype).cpu().numpy()
    ref = _oracle(d, w_dtype, np.arange(T))
    err, rms = parity.rel_err(out, ref)
    _say("dense small", w_dtype, T, "max|err|/rms", err)
    assert err <= parity.TOL[w_dtype]


def _fp8_every_row(d, bar=True):
    """FP8 dense layer through the every-row check (fullcheck.py): the layer is one expert that
    every token takes with weight 1, so the MoE rules apply with E = K = 1. bar: also hold every
    token other than the counted near-flip tokens to the FP8 bar against the pure oracle."""
    import fullcheck
    T, H, F = d["T"], d["hidden"], d["d_ff"]
    cfg = bm.make_cfg(H, 1, 1, 1, 1, F, 1.0, bm.BEAM_BF16, bm.BEAM_FP8_E4M3, bm.BEAM_F32)
    ws = torch.empty(bm.dense_workspace_bytes(H, F, bm.BEAM_FP8_E4M3, T), dtype=torch.uint8,
                     device="cuda")
    out = bm.dense_mlp(d["x"], d["w_gate_up"], d["w_down"], w_gate_up_scale=d["w_gate_up_scale"],
                       w_down_scale=d["w_down_scale"], workspace=ws)
    torch.cuda.synchronize()
    ex = fullcheck.expert_f64(d["w_gate_up"], d["w_down"], F, d["w_gate_up_scale"],
                              d["w_down_scale"])
    st = fullcheck.read_state(ws, cfg, T, True, dense=True)
    parts = st["y"].numel() // (T * H)
    stats = fullcheck.check_batch(out, d["x"], np.zeros((T, 1), dtype=np.int64), np.ones((T, 1)),
                                  st, lambda e: ex, "fp8", 1, say=_say, y_parts=parts)
    assert stats["tokens_checked"] == T
    assert stats["near_flip_tokens"] <= max(2, T // 50), stats
    if bar:
        assert stats["err_out_pure"] <= parity.TOL["fp8"], stats
    return stats, parts


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


def test_beam_dense_fp8_every_token():
    """Beam's dense layer with FP8 weights (5120 x 20480): every token of a 2048-token batch (the
    down GEMM splits K into 4 parts) through the every-row check, at the FP8 bar against the pure
    oracle except counted near-flip tokens; and T = 32 (decode kernels) likewise."""
    _say("generating Beam dense layer (5120 x 20480, FP8) on cuda:0")
    d = synthgen.make_dense(2048, w_dtype="fp8", device="cuda")
    torch.cuda.synchronize()
    stats, parts = _fp8_every_row(d)
    _say("Beam dense FP8 T=2048, down K parts", parts, stats)
    assert parts == 4
    d32 = dict(d)
    d32["x"] = d["x"][:32].contiguous()
    d32["T"] = 32
    _fp8_every_row(d32)
