"""beam_moe_forward_noalloc, the forward that allocates nothing (its workspace is the library's own
per-GPU device array), against beam_moe_forward on a caller workspace: identical outputs, routes and
weights, bit for bit, over consecutive calls whose batches shrink (the array keeps the previous
call's contents), on the tiled and the decode paths, bf16 and FP8; and an oversized batch rejected
before anything is launched."""
import numpy as np
import pytest
import torch

import routing_grouped_expert_fp32_amd as bm
import synthgen

pytestmark = pytest.mark.gpu
SH = synthgen.BEAM_SHAPE


def _pair(W, wl_name, T, cfg):
    d = synthgen.make_inputs(wl_name, device="cuda", T=T, with_experts=False)
    kw = {}
    if "w_gate_up_scale" in W:
        kw = dict(w_gate_up_scale=W["w_gate_up_scale"], w_down_scale=W["w_down_scale"])
    ids_a = torch.empty((T, SH.topk), dtype=torch.int32, device="cuda")
    ids_b = torch.empty_like(ids_a)
    w_a = torch.empty((T, SH.topk), dtype=torch.float32, device="cuda")
    w_b = torch.empty_like(w_a)
    ref = bm.forward(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg,
                     topk_ids_out=ids_a, topk_w_out=w_a, **kw)
    got = bm.forward_noalloc(d["x"], W["w_router"], d["bias"], W["w_gate_up"], W["w_down"], cfg,
                             topk_ids_out=ids_b, topk_w_out=w_b, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a.view(torch.int32), w_b.view(torch.int32))
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), T
    print("no-alloc forward equals forward, T =", T, flush=True)


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_noalloc_equals_forward_on_shrinking_batches(w_dtype):
    name = "fp8_decode" if w_dtype == "fp8" else "decode"
    W = synthgen.make_inputs(name, device="cuda", T=1)
    cfg = bm.WorkloadCfg.of(SH, "bf16", w_dtype)
    for T in (256, 64, 7):   # tiled experts, then the small-batch paths
        _pair(W, name, T, cfg)
    del W


def test_noalloc_rejects_batches_past_its_workspace():
    cfg = bm.WorkloadCfg.of(SH, "bf16", "bf16")
    T = 400
    assert bm.workspace_bytes(cfg, T) > 64 << 20
    x = torch.zeros((T, SH.hidden), dtype=torch.bfloat16, device="cuda")
    w_r = torch.zeros((SH.n_experts, SH.hidden), dtype=torch.float32, device="cuda")
    bias = torch.zeros(SH.n_experts, dtype=torch.float32, device="cuda")
    wgu = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")   # never read: rejected first
    out = torch.full((T, SH.hidden), 7.0, device="cuda")
    with pytest.raises(bm.BeamError) as ei:
        bm.forward_noalloc(x, w_r, bias, wgu, wgu, cfg, out=out)
    assert ei.value.status == 6   # BEAM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all()     # nothing was launched
