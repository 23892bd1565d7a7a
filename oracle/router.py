"""Oracle router: FP64 logits, sigmoid scores, group-limited top-k, routing weights, cut margins.

Test infrastructure only (see the package docstring).

Method ([V] §MoE and residual stream; [H] §专家混合; [N] §1; [S] §Dense Layers and Grouped MoE
Routing): the router projects the token onto the E experts (FP32 weights in the model; here every
product and sum is taken in float64, so the logits are exact up to ~1e-16 relative). Each expert's
score is the sigmoid of its logit; adding the expert correction bias gives the selection score b.
The E experts form G equal, contiguous groups. A group's score is the sum of its two largest b.
The Gk best groups are kept; the K experts with the largest b among the kept groups' members
(no per-group quota) are selected. The weights renormalise the *unbiased* sigmoid scores of the
selected experts and multiply by the routed scale (2.5 for Beam).

Readings where the pages are silent:
  * ties (equal float64 values) go to the lower group index and to the lower expert index;
  * non-kept experts are excluded from the top-K (not given score 0);
  * the bias enters group ranking and expert choice only, never the weights;
  * ids are returned in selection order (b descending, ties to the lower id).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class RouteResult:
    ids: np.ndarray            # [T][K] int64, selection order
    weights: np.ndarray        # [T][K] float64, sum = routed_scale
    s: np.ndarray              # [T][E] sigmoid scores
    b: np.ndarray              # [T][E] selection scores s + bias
    group_score: np.ndarray    # [T][G]
    kept_groups: np.ndarray    # [T][Gk], best first
    margin_group: np.ndarray   # [T]  score(Gk-th kept) - score(best dropped); inf if none dropped
    margin_expert: np.ndarray  # [T]  b(K-th chosen) - b(best unchosen candidate); inf if none

    @property
    def margin(self) -> np.ndarray:
        """Smallest cut margin per token: how far the choice is from flipping."""
        return np.minimum(self.margin_group, self.margin_expert)


def to_f64(a) -> np.ndarray:
    """Exact float64 copy of a torch tensor / array in fp32, bf16 or fp64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def logits(x, w_router) -> np.ndarray:
    """logits[t][e] = sum_h x[t][h] * W_r[e][h] in float64. W_r is stored [E][H] (the transpose of
    the pages' H x E router matrix), so both operands run along H."""
    return to_f64(x) @ to_f64(w_router).T


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def select(b: np.ndarray, n_groups: int, topk_groups: int, topk: int):
    """Group-limited selection on the selection scores b [T][E].

    Returns (ids [T][K], group_score [T][G], kept [T][Gk], margin_group [T], margin_expert [T]).
    """
    b = np.asarray(b, dtype=np.float64)
    T, E = b.shape
    G = n_groups
    if E % G or topk_groups > G or topk > topk_groups * (E // G) or min(G, topk_groups, topk) < 1:
        raise ValueError("inconsistent routing configuration")
    gs = E // G
    grouped = b.reshape(T, G, gs)
    two_largest = np.sort(grouped, axis=2)[:, :, gs - 2:] if gs >= 2 else grouped
    group_score = two_largest.sum(axis=2)

    # best groups first; a stable sort on the negated score keeps equal scores in index order
    g_order = np.argsort(-group_score, axis=1, kind="stable")
    kept = g_order[:, :topk_groups]
    g_sorted = np.take_along_axis(group_score, g_order, axis=1)
    margin_group = (g_sorted[:, topk_groups - 1] - g_sorted[:, topk_groups]
                    if topk_groups < G else np.full(T, np.inf))

    member = np.zeros((T, G), dtype=bool)
    np.put_along_axis(member, kept, True, axis=1)
    cand = np.repeat(member, gs, axis=1)                       # expert e belongs to group e // gs
    masked = np.where(cand, b, -np.inf)
    e_order = np.argsort(-masked, axis=1, kind="stable")
    ids = e_order[:, :topk]
    n_cand = topk_groups * gs
    e_sorted = np.take_along_axis(masked, e_order, axis=1)
    margin_expert = (e_sorted[:, topk - 1] - e_sorted[:, topk] if topk < n_cand
                     else np.full(T, np.inf))
    return ids.astype(np.int64), group_score, kept, margin_group, margin_expert


def weights(s: np.ndarray, ids: np.ndarray, routed_scale: float) -> np.ndarray:
    """w_k = routed_scale * s[e_k] / sum_j s[e_j] (unbiased scores of the chosen experts)."""
    chosen = np.take_along_axis(np.asarray(s, dtype=np.float64), ids, axis=1)
    return routed_scale * chosen / chosen.sum(axis=1, keepdims=True)


def route(x, w_router, bias, n_groups: int, topk_groups: int, topk: int,
          routed_scale: float) -> RouteResult:
    """Full routing of x [T][H] with router weights [E][H] and correction bias [E]."""
    z = logits(x, w_router)
    s = sigmoid(z)
    b = s + to_f64(bias)[None, :]
    ids, gscore, kept, mg, me = select(b, n_groups, topk_groups, topk)
    w = weights(s, ids, routed_scale)
    return RouteResult(ids, w, s, b, gscore, kept, mg, me)


def route_cfg(inputs: dict) -> RouteResult:
    """route() on a synthgen input dict."""
    sh = inputs["workload"].shape
    return route(inputs["x"], inputs["w_router"], inputs["bias"], sh.n_groups, sh.topk_groups,
                 sh.topk, sh.routed_scale)
