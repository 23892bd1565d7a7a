"""Oracle of the sublayer boundary that follows the MoE: output RMSNorm, depth-scaled residual add,
next input RMSNorm (test infrastructure only; see the package docstring).

Sources: [V] §MoE and residual stream (every sublayer has an RMSNorm before and after it; the n-th
residual add computes h <- sqrt((n-1)/n) h + x / sqrt(n)); [S] §Sandwich Normalization and
Depth-Scaled Residuals (the branch and the residual are scaled by depth-derived coefficients and
both rounded to the activation dtype before the addition); [V] §Agent-driven optimization item 1
(FP32 math with BF16 rounding points) and item 3 (after the MoE the boundary also combines the
top-8 outputs); [H] §残差流 (the input embedding counts as add 1; the two weights' squares sum to 1).

Readings (the pages leave these open): RMSNorm(v) = v * gamma / sqrt(mean(v^2) + eps) with one
rounding of the product to bf16; eps is a parameter (unstated on the pages); the sublayer output is
taken in the activation dtype (bf16) before its norm. Computed in float64 with the bf16 rounding
points of the definition (codecs.bf16_round).
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round
from .router import to_f64


def rmsnorm(v, gamma, eps: float) -> np.ndarray:
    """v * gamma / sqrt(mean(v^2) + eps) along the last axis, float64, unrounded."""
    v = to_f64(v)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * to_f64(gamma)


def residual_coefficients(n: int):
    """(alpha, beta) of the n-th residual add: sqrt((n-1)/n) and 1/sqrt(n)."""
    return float(np.sqrt((n - 1) / n)), float(1.0 / np.sqrt(n))


def boundary(y, h, gamma_post, gamma_next, n: int, eps: float, return_parts: bool = False):
    """(h_out, x_next) for sublayer output y [T][H] and residual stream h [T][H] (bf16 values)."""
    u = bf16_round(to_f64(y))
    p = bf16_round(rmsnorm(u, gamma_post, eps))
    alpha, beta = residual_coefficients(n)
    a = bf16_round(alpha * to_f64(h))
    b = bf16_round(beta * p)
    h_out = bf16_round(a + b)
    x_next = bf16_round(rmsnorm(h_out, gamma_next, eps))
    if return_parts:
        return h_out, x_next, {"u": u, "p": p, "a": a, "b": b}
    return h_out, x_next
