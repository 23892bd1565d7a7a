"""GPU routing on configurations other than Beam's and the small test model, against the oracle:
no group limit with the largest top-k (16, the most slots the combine sums), one expert per group,
an uneven keep count, and a single expert per token. Each runs the forward on all three routing
paths (T = 5: selection fused with align; T = 300: hidden-chunk partial logits; T = 1500: the
one-pass router): ids exact except counted near-ties, weights within 1e-5 of the oracle's, and the
output of sampled tokens at the bf16 bar."""
import dataclasses

import numpy as np
import pytest
import torch

import parity
import routing_grouped_expert_fp32_amd as bm
import synthgen
from oracle import router

pytestmark = pytest.mark.gpu

CONFIGS = {
    "E256-G1-K16": dict(n_experts=256, n_groups=1, topk_groups=1, topk=16),
    "E64-G64-K8": dict(n_experts=64, n_groups=64, topk_groups=8, topk=8),
    "E128-G16-K6": dict(n_experts=128, n_groups=16, topk_groups=3, topk=6),
    "E16-G4-K1": dict(n_experts=16, n_groups=4, topk_groups=2, topk=1),
}


@pytest.mark.parametrize("T", [5, 300, 1500])
@pytest.mark.parametrize("name", list(CONFIGS))
def test_routing_config(name, T):
    shape = synthgen.BeamShape(hidden=512, d_ff=256, **CONFIGS[name])
    wl = dataclasses.replace(synthgen.WORKLOADS["tiny"], name=f"route_{name}_{T}", T=T,
                             shape=shape, x_dtype="bf16", w_dtype="bf16", sigma_w=0.05)
    print("routing config", name, "T =", T, flush=True)
    d = synthgen.make_inputs(wl, device="cuda")
    cfg = bm.WorkloadCfg.of(shape, "bf16", "bf16")
    ids = torch.empty((T, shape.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, shape.topk), dtype=torch.float32, device="cuda")
    out = bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], cfg,
                     topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    r = router.route(d["x"].cpu(), d["w_router"].cpu(), d["bias"].cpu(), shape.n_groups,
                     shape.topk_groups, shape.topk, shape.routed_scale)
    ids_c = ids.cpu().numpy()
    rc = parity.check_routing(ids_c, w.cpu().numpy(), r)
    print(name, T, "near ties", len(rc["near_ties"]), "max|dw|", rc["max_dw"], flush=True)
    assert rc["ok"], rc
    assert len(rc["near_ties"]) <= max(1, T // 100), rc
    np.testing.assert_allclose(w.cpu().numpy().sum(axis=1), shape.routed_scale, rtol=1e-5)
    get = parity.expert_loader(d["w_gate_up"], d["w_down"], shape.d_ff)
    tokens = np.unique(np.linspace(0, T - 1, min(T, 16)).astype(np.int64))
    err, _ = parity.check_outputs(out.cpu().numpy(), d["x"], ids_c, r, shape.routed_scale, get,
                                  "bf16", tokens)
    print(name, T, "max|err|/rms", err, flush=True)
    assert err <= parity.TOL["bf16"]
