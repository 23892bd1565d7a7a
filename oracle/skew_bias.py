"""Finds the correction-bias offset delta of the skewed workload and stores it.

Test infrastructure only (see the package docstring). The skewed workload (T = 32768 tokens) puts
bias delta on 16 "hot" experts (synthgen.hot_set) and 0 elsewhere; delta is chosen by bisection
under this oracle's FP64 router so that 40 % +- 0.5 % of the T * 8 slots land on the hot set.

    python -m oracle.skew_bias            # writes tests/golden/skew_bias.json
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthgen  # noqa: E402
from oracle import router  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "skew_bias.json")


def hot_fraction(s: np.ndarray, delta: float, hot: list, sh) -> float:
    bias = np.zeros(sh.n_experts)
    bias[hot] = float(np.float32(delta))        # the bias tensor is fp32
    ids, *_ = router.select(s + bias[None, :], sh.n_groups, sh.topk_groups, sh.topk)
    return float(np.isin(ids, hot).mean())


def find_delta(T: int | None = None, iters: int = 40) -> dict:
    wl = synthgen.WORKLOADS["skew"]
    sh = wl.shape
    T = wl.T if T is None else T
    d = synthgen.make_inputs(wl, T=T, with_experts=False, skew_delta=0.0)
    s = router.sigmoid(router.logits(d["x"], d["w_router"]))
    hot = synthgen.hot_set(wl.n_hot, sh.n_experts, wl.seed)
    target, tol = synthgen.skew_hot_fraction_target()
    lo, hi = 0.0, 1.0
    f_lo, f_hi = hot_fraction(s, lo, hot, sh), hot_fraction(s, hi, hot, sh)
    if not f_lo < target < f_hi:
        raise RuntimeError(f"target {target} not bracketed: {f_lo} .. {f_hi}")
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        f = hot_fraction(s, mid, hot, sh)
        if abs(f - target) <= tol / 4:
            lo = hi = mid
            break
        if f < target:
            lo = mid
        else:
            hi = mid
    delta = float(np.float32(0.5 * (lo + hi)))
    frac = hot_fraction(s, delta, hot, sh)
    if abs(frac - target) > tol:
        raise RuntimeError(f"bisection ended at fraction {frac}")
    return {"workload": "skew", "T": T, "hot_experts": hot, "delta": delta,
            "hot_fraction": frac, "target": target, "tolerance": tol,
            "made_by": "python -m oracle.skew_bias"}


def main():
    res = find_delta()
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
