"""GPU parity on non-Beam shapes that take the other kernel variants: a d_ff whose quarter rows are
not whole K-split batches (the column-tiled small-block kernel), the tiled kernel on a small
model, and a mid-size model whose K-split decode loops run an even and an odd number of batches
per wave, in bf16 and FP8, every token against the CPU oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import router

pytestmark = pytest.mark.gpu

# H 512, 32 experts in 8 groups (keep 2), top-4, d_ff 768: down rows are 1536 B (bf16) / 768 B
# (FP8), whose quarters (384 B / 192 B) are not whole K-split batches
SHAPE = synthgen.BeamShape(hidden=512, n_experts=32, n_groups=8, topk_groups=2, topk=4, d_ff=768)


# H 2048, d_ff 1536: each of the 4 K-split waves runs 4 batches of gate/up rows (4096 B bf16 /
# 2048 B FP8) and 3 of down rows (3072 B / 1536 B), so the decode loop ends on the even path (a
# last trip whose next-batch loads hit empty buffers) for gate/up and on the odd tail for down
MID_SHAPE = synthgen.BeamShape(hidden=2048, n_experts=32, n_groups=8, topk_groups=2, topk=4,
                               d_ff=1536)


def _wl(w_dtype, T, shape=SHAPE):
    return dataclasses.replace(synthgen.WORKLOADS["tiny"], name=f"shape_{w_dtype}_{T}", T=T,
                               shape=shape, x_dtype="bf16", w_dtype=w_dtype, sigma_w=0.05)


@pytest.mark.parametrize("w_dtype,T,shape", [("bf16", 24, SHAPE), ("bf16", 200, SHAPE),
                                             ("fp8", 24, SHAPE), ("fp8", 200, SHAPE)],
                         ids=["bf16-24", "bf16-200", "fp8-24", "fp8-200"])
def test_small_model_all_tokens(w_dtype, T, shape):
    wl = _wl(w_dtype, T, shape)
    print("shape test", w_dtype, "T =", T, "hidden", shape.hidden, "d_ff", shape.d_ff, flush=True)
    d = synthgen.make_inputs(wl, device="cuda")
    cfg = bm.WorkloadCfg.of(shape, "bf16", w_dtype)
    ids = torch.empty((T, shape.topk), dtype=torch.int32, device="cuda")
    kw = {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=d["w_gate_up_scale"], w_down_scale=d["w_down_scale"])
    out = bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], cfg,
                     topk_ids_out=ids, **kw)
    torch.cuda.synchronize()
    r = router.route(d["x"].cpu(), d["w_router"].cpu(), d["bias"].cpu(), shape.n_groups,
                     shape.topk_groups, shape.topk, shape.routed_scale)
    ids_c = ids.cpu().numpy()
    rc = parity.check_routing(ids_c, router.weights(r.s, ids_c.astype(np.int64), 2.5), r)
    assert not rc["failures"], rc
    get = parity.expert_loader(d["w_gate_up"], d["w_down"], shape.d_ff,
                               d.get("w_gate_up_scale"), d.get("w_down_scale"))
    err, rms = parity.check_outputs(out.cpu().numpy(), d["x"], ids_c, r, shape.routed_scale, get,
                                    w_dtype, np.arange(T))
    print(w_dtype, T, "max|err|/rms", err, flush=True)
    assert err <= parity.TOL[w_dtype]


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_small_model_multi_block_experts(w_dtype):
    """T = 3000 on the small model: ~375 rows per expert, so every expert spans two 320-row tiled
    blocks (a full one and a partial one). Every row and every token through the every-row check
    (fullcheck.py): h of each row within its admissible roundings, codes bit for bit, each slot's
    output against its own h, and every token at the bar except counted near-flip tokens."""
    import fullcheck
    T = 3000
    wl = _wl(w_dtype, T)
    print("multi-block experts", w_dtype, "T =", T, flush=True)
    d = synthgen.make_inputs(wl, device="cuda")
    cfg = bm.WorkloadCfg.of(SHAPE, "bf16", w_dtype)
    ids = torch.empty((T, SHAPE.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    kw = {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=d["w_gate_up_scale"], w_down_scale=d["w_down_scale"])
    out = bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], cfg,
                     topk_ids_out=ids, workspace=ws, **kw)
    torch.cuda.synchronize()
    ids_c = ids.cpu().numpy().astype(np.int64)
    counts = np.bincount(ids_c.ravel(), minlength=SHAPE.n_experts)
    assert (counts > 320).sum() >= SHAPE.n_experts // 2, counts
    r = router.route(d["x"].cpu(), d["w_router"].cpu(), d["bias"].cpu(), SHAPE.n_groups,
                     SHAPE.topk_groups, SHAPE.topk, SHAPE.routed_scale)
    rc = parity.check_routing(ids_c, router.weights(r.s, ids_c, 2.5), r)
    assert not rc["failures"], rc
    fp8 = w_dtype == "fp8"

    def get(e):
        return fullcheck.expert_f64(d["w_gate_up"][e], d["w_down"][e], SHAPE.d_ff,
                                    d["w_gate_up_scale"][e] if fp8 else None,
                                    d["w_down_scale"][e] if fp8 else None)
    st = fullcheck.read_state(ws, cfg, T, fp8)
    stats = fullcheck.check_batch(out, d["x"], ids_c, router.weights(r.s, ids_c, 2.5), st, get,
                                  w_dtype, SHAPE.n_experts)
    assert stats["tokens_checked"] == T
    assert stats["err_out_pure"] <= parity.TOL[w_dtype], stats
    assert stats["near_flip_tokens"] <= T // 50, stats


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_mid_model_decode_loops(w_dtype):
    """T = 40 on the mid-size model (decode-sized blocks, so the K-split kernels): every row and
    every token through the every-row check, as for the multi-block case."""
    import fullcheck
    T = 40
    wl = _wl(w_dtype, T, MID_SHAPE)
    print("mid model", w_dtype, "T =", T, flush=True)
    d = synthgen.make_inputs(wl, device="cuda")
    cfg = bm.WorkloadCfg.of(MID_SHAPE, "bf16", w_dtype)
    ids = torch.empty((T, MID_SHAPE.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    kw = {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=d["w_gate_up_scale"], w_down_scale=d["w_down_scale"])
    out = bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], cfg,
                     topk_ids_out=ids, workspace=ws, **kw)
    torch.cuda.synchronize()
    ids_c = ids.cpu().numpy().astype(np.int64)
    r = router.route(d["x"].cpu(), d["w_router"].cpu(), d["bias"].cpu(), MID_SHAPE.n_groups,
                     MID_SHAPE.topk_groups, MID_SHAPE.topk, MID_SHAPE.routed_scale)
    rc = parity.check_routing(ids_c, router.weights(r.s, ids_c, 2.5), r)
    assert not rc["failures"], rc
    fp8 = w_dtype == "fp8"

    def get(e):
        return fullcheck.expert_f64(d["w_gate_up"][e], d["w_down"][e], MID_SHAPE.d_ff,
                                    d["w_gate_up_scale"][e] if fp8 else None,
                                    d["w_down_scale"][e] if fp8 else None)
    st = fullcheck.read_state(ws, cfg, T, fp8)
    stats = fullcheck.check_batch(out, d["x"], ids_c, router.weights(r.s, ids_c, 2.5), st, get,
                                  w_dtype, MID_SHAPE.n_experts)
    print(w_dtype, stats, flush=True)
    assert stats["tokens_checked"] == T
    assert stats["err_out_pure"] <= parity.TOL[w_dtype], stats
    assert stats["near_flip_tokens"] <= 2, stats
