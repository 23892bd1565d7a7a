"""Runtime behaviour of the library through the C ABI: a forward step captured in a HIP graph replays
to the eager result (a call launches kernels on the caller's stream and nothing else: no allocation,
memset or synchronisation), the stage-timing mask records only the selected stages, and the
BEAM_MOE_SYNC_CHECK debugging mode leaves the results unchanged."""
import dataclasses

import pytest
import torch

import routing_grouped_expert_fp32_amd as bm
import synthgen

pytestmark = pytest.mark.gpu

# H 512, 32 experts in 8 groups (keep 2), top-4, d_ff 768: T=8 and T=32 take the small-block
# kernels, T=700 (~87 rows per expert) the tiled ones
SHAPE = synthgen.BeamShape(hidden=512, n_experts=32, n_groups=8, topk_groups=2, topk=4, d_ff=768)


def _case(w_dtype, T):
    wl = dataclasses.replace(synthgen.WORKLOADS["tiny"], name=f"runtime_{w_dtype}_{T}", T=T,
                             shape=SHAPE, x_dtype="bf16", w_dtype=w_dtype, sigma_w=0.05)
    d = synthgen.make_inputs(wl, device="cuda")
    cfg = bm.WorkloadCfg.of(SHAPE, "bf16", w_dtype)
    kw = {}
    if w_dtype == "fp8":
        kw = dict(w_gate_up_scale=d["w_gate_up_scale"], w_down_scale=d["w_down_scale"])
    ws = torch.empty(bm.workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, SHAPE.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, SHAPE.topk), dtype=torch.int32, device="cuda")

    def run(stream=None):
        bm.forward(d["x"], d["w_router"], d["bias"], d["w_gate_up"], d["w_down"], cfg, out=out,
                   topk_ids_out=ids, workspace=ws, stream=stream, **kw)

    return run, out, ids


@pytest.mark.parametrize("w_dtype,T",
                         [("bf16", 8), ("fp8", 32), ("bf16", 700), ("fp8", 700), ("bf16", 1100)])
def test_graph_replay_equals_eager(w_dtype, T):
    print("graph capture", w_dtype, "T =", T, flush=True)
    run, out, ids = _case(w_dtype, T)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run(s)
    torch.cuda.synchronize()
    ref, ref_ids = out.clone(), ids.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    torch.cuda.synchronize()
    for i in range(3):   # eager work and a synchronisation between the replays
        out.fill_(float("nan"))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(ids, ref_ids), f"replay {i}"


def test_timing_stage_mask():
    run, _, _ = _case("bf16", 16)
    run()
    torch.cuda.synchronize()
    bm.timing_enable(True, stages=["gate_up"])
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    bm.timing_enable(False)
    st = bm.timing_collect()
    assert st["gate_up"][1] == 3 and st["gate_up"][0] > 0
    assert all(n == 0 for k, (_, n) in st.items() if k != "gate_up"), st
    bm.timing_enable(True)
    run()
    torch.cuda.synchronize()
    bm.timing_enable(False)
    st = bm.timing_collect()
    # up to 16 tokens the selection and the align are one launch (recorded as router_select)
    for k in ("router_logits", "router_select", "gate_up", "down", "combine"):
        assert st[k][1] == 1, (k, st)
    assert st["moe_align"][1] == 0, st
    run2, _, _ = _case("bf16", 17)
    bm.timing_enable(True)
    run2()
    torch.cuda.synchronize()
    bm.timing_enable(False)
    st = bm.timing_collect()
    for k in ("router_logits", "router_select", "moe_align", "gate_up", "down", "combine"):
        assert st[k][1] == 1, (k, st)
    # past 1024 tokens bf16 activations take the one-pass router, after the split of the router
    # weights (both recorded as router_logits)
    run3, _, _ = _case("bf16", 1100)
    bm.timing_enable(True)
    run3()
    torch.cuda.synchronize()
    bm.timing_enable(False)
    st = bm.timing_collect()
    assert st["router_logits"][1] == 2, st
    for k in ("moe_align", "gate_up", "down", "combine"):
        assert st[k][1] == 1, (k, st)
    assert st["router_select"][1] == 0, st


def test_two_streams_with_their_own_workspaces():
    """Calls on two streams at once, each with its own workspace, give the results of serial calls
    (the library keeps no state between calls besides the timing records)."""
    run_a, out_a, ids_a = _case("bf16", 700)
    run_b, out_b, ids_b = _case("fp8", 40)
    run_a()
    run_b()
    torch.cuda.synchronize()
    ref_a, ref_b = out_a.clone(), out_b.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(3):
        out_a.fill_(float("nan"))
        out_b.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            run_a(s1)
        with torch.cuda.stream(s2):
            run_b(s2)
        torch.cuda.synchronize()
        assert torch.equal(out_a, ref_a) and torch.equal(out_b, ref_b), f"round {i}"


def test_sync_check_mode_gives_the_same_results(tmp_path):
    """BEAM_MOE_SYNC_CHECK=1 (a stream synchronisation after every launch, failures reported by
    stage) changes nothing in the results: a child process with it set writes the same bits."""
    import os
    import subprocess
    import sys
    code = (
        "import sys, torch\n"
        "sys.path.insert(0, sys.argv[1])\n"
        "import test_gpu_runtime as t\n"
        "run, out, ids = t._case('bf16', 300)\n"
        "run(); torch.cuda.synchronize()\n"
        "torch.save({'out': out.cpu(), 'ids': ids.cpu()}, sys.argv[2])\n")
    here = os.path.dirname(os.path.abspath(__file__))
    res = {}
    for mode in ("0", "1"):
        path = str(tmp_path / f"sync_{mode}.pt")
        env = dict(os.environ, BEAM_MOE_SYNC_CHECK=mode,
                   PYTHONPATH=os.pathsep.join([os.path.dirname(here), here,
                                               os.environ.get("PYTHONPATH", "")]))
        r = subprocess.run([sys.executable, "-c", code, here, path], env=env, capture_output=True,
                           text=True, timeout=240)
        assert r.returncode == 0, r.stderr[-2000:]
        res[mode] = torch.load(path, weights_only=True)
    assert torch.equal(res["0"]["ids"], res["1"]["ids"])
    assert torch.equal(res["0"]["out"].view(torch.int32), res["1"]["out"].view(torch.int32))
