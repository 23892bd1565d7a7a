"""Parity helpers: compare the HIP path's routing and output with the CPU oracle (tests only).

Rules (the block's acceptance bar):
  * expert ids: per token, the chosen SET must equal the oracle's; a token whose oracle cut margin
    (group cut or expert cut, FP64) is below 1e-6 may differ — it is counted as a near-tie, not a
    failure. The GPU decides in FP32, the oracle in FP64; near a cut both are correct choices.
  * the GPU order must be by descending oracle score up to that same 1e-6 margin;
  * routing weights on set-matching tokens: |dw| <= 1e-5;
  * outputs: max|out - ref| / rms(ref) <= 1e-2 (bf16 experts), 5e-2 (fp8), 1e-4 (fp32, where the
    expected figure is ~1e-6). Near-tie tokens are compared against the oracle recomputed with the
    GPU's ids (and oracle weights for those ids).
"""
from __future__ import annotations

import os

import numpy as np
import torch

from oracle import experts, router

_OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def say(*a):
    """Progress line of a long check: printed, and appended to test_progress.log in the run-output
    folder at the repository root when that folder exists (a captured test's progress is then
    still visible while it runs)."""
    msg = " ".join(str(x) for x in a)
    print(msg, flush=True)
    if os.path.isdir(_OUT):
        with open(os.path.join(_OUT, "test_progress.log"), "a") as f:
            f.write(msg + "\n")


MARGIN = 1e-6
TOL = {"bf16": 1e-2, "fp8": 5e-2, "f32": 1e-4}


def check_routing(ids_gpu, w_gpu, r: router.RouteResult, tokens=None, w_tol=1e-5):
    ids_gpu = np.asarray(ids_gpu, dtype=np.int64)
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    T = ids_gpu.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    near, fail, order_bad = [], [], []
    max_dw = 0.0
    for i, t in enumerate(tokens):
        g, o = ids_gpu[i], r.ids[t]
        if len(set(g.tolist())) != len(g) or g.min() < 0 or g.max() >= r.b.shape[1]:
            fail.append(int(t))
            continue
        if sorted(g) != sorted(o):
            (near if r.margin[t] < MARGIN else fail).append(int(t))
            continue
        bg = r.b[t][g]
        if np.any(bg[:-1] < bg[1:] - MARGIN):
            order_bad.append(int(t))
        ow = dict(zip(o.tolist(), r.weights[t].tolist()))
        max_dw = max(max_dw, max(abs(w_gpu[i][k] - ow[int(g[k])]) for k in range(len(g))))
    return {"near_ties": near, "failures": fail, "order_bad": order_bad, "max_dw": max_dw,
            "ok": not fail and not order_bad and max_dw <= w_tol}


def expert_loader(w_gate_up, w_down, d_ff, gu_scale=None, dn_scale=None, cache=None):
    """get_expert(e) for the oracle, copying one expert's stored tensors to the host."""
    cache = {} if cache is None else cache

    def get(e):
        if e not in cache:
            cache[e] = experts.split_expert(
                w_gate_up[e].cpu(), w_down[e].cpu(), d_ff,
                None if gu_scale is None else gu_scale[e].cpu(),
                None if dn_scale is None else dn_scale[e].cpu())
        return cache[e]
    return get


def oracle_out(x_rows, ids_rows, w_rows, get_expert, contract):
    return experts.forward_expert_major(x_rows, ids_rows, w_rows, get_expert, contract)


def rel_err(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(out - ref)) / rms), float(rms)


def check_outputs(out_gpu, x, ids_gpu, rres: router.RouteResult, scale, get_expert, contract,
                  tokens, arrays=False):
    """Output parity on `tokens` (indices into the full batch). Tokens whose id set matches use the
    oracle's routing; near-tie tokens use the GPU's ids with oracle weights for them. Returns
    (max|err|/rms, rms), and with arrays=True also the GPU and oracle outputs compared."""
    tokens = np.asarray(tokens)
    ids_gpu = np.asarray(ids_gpu, dtype=np.int64)[tokens]
    use_ids = rres.ids[tokens].copy()
    for i, t in enumerate(tokens):
        if sorted(ids_gpu[i]) != sorted(rres.ids[t]):
            use_ids[i] = ids_gpu[i]
    use_w = router.weights(rres.s[tokens], use_ids, scale)
    xr = router.to_f64(x[torch.from_numpy(tokens).to(x.device)])
    ref = oracle_out(xr, use_ids, use_w, get_expert, contract)
    got = np.asarray(out_gpu, dtype=np.float64)
    if got.shape[0] != len(tokens):
        got = got[tokens]
    if arrays:
        return rel_err(got, ref) + (got, ref)
    return rel_err(got, ref)
