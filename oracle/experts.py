"""Oracle experts and combine under the three numerics contracts (fp32, bf16, fp8).

Test infrastructure only (see the package docstring).

Expert e is a SwiGLU MLP without biases ([H] §专家混合: d_ff 2560, ~39M parameters = 3 matrices of
5120 x 2560; [N] §1): h = silu(G_e x) * (U_e x), y = D_e h, silu(z) = z * sigmoid(z).
Storage reading: the fused gate/up tensor of an expert is [2F][H] with gate rows [0, F) and up rows
[F, 2F); the down tensor is [H][F]. Every row runs along the contracted dimension.

Contracts (the rounding points are those the BF16 expert kernels keep, [S] §BF16 MoE Kernel
Optimization; the product silu(gate)*up is an FP32 quantity of the model, [H] §残差流):
  "fp32": no rounding anywhere (float64 throughout).
  "bf16": g, u = bf16(G x), bf16(U x); h = bf16(silu(g) * u); y = D h exact; the FP32 routing weight
          multiplies y before any rounding; contributions and out stay un-rounded.
  "fp8":  x is quantised per token and h per row with codecs.quant_rows_fp8; weights arrive as E4M3
          codes with fp32 per-output-channel scales; g = s_x * s_w[j] * (codes . codes), then the bf16
          steps as above; y = s_h * s_d[n] * (codes . codes).
Combine ([V] §MoE and residual stream; [H] §专家混合): out[t] = sum over k = 0..K-1, in that order, of
w[t][k] * y[t][k]; there is no shared expert.
"""
from __future__ import annotations

from typing import Callable

import numpy as np

from .codecs import bf16_round, e4m3_decode, quant_rows_fp8
from .router import to_f64


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_mlp(x_rows: np.ndarray, ex: dict, contract: str) -> np.ndarray:
    """y [n][H] for token rows x_rows [n][H] through one expert.

    `ex` holds float64 matrices "gate" [F][H], "up" [F][H], "down" [H][F]; for the fp8 contract
    these are the *decoded codes* and `ex` also holds "gate_scale" [F], "up_scale" [F],
    "down_scale" [H]. For the fp8 contract x_rows must be the bf16 token values (float64 copies).
    """
    x = to_f64(x_rows)
    if contract == "fp32":
        g = x @ ex["gate"].T
        u = x @ ex["up"].T
        return (silu(g) * u) @ ex["down"].T
    if contract == "bf16":
        g = bf16_round(x @ ex["gate"].T)
        u = bf16_round(x @ ex["up"].T)
        h = bf16_round(silu(g) * u)
        return h @ ex["down"].T
    if contract == "fp8":
        qx, sx = quant_rows_fp8(x)
        xd = e4m3_decode(qx)
        sx = sx.astype(np.float64)[:, None]
        g = bf16_round(sx * ex["gate_scale"][None, :] * (xd @ ex["gate"].T))
        u = bf16_round(sx * ex["up_scale"][None, :] * (xd @ ex["up"].T))
        h = bf16_round(silu(g) * u)
        qh, sh = quant_rows_fp8(h)
        hd = e4m3_decode(qh)
        return sh.astype(np.float64)[:, None] * ex["down_scale"][None, :] * (hd @ ex["down"].T)
    raise ValueError(f"unknown contract {contract!r}")


def combine(contrib: np.ndarray) -> np.ndarray:
    """out[t] = contrib[t][0] + contrib[t][1] + ... in k order (contrib [T][K][H])."""
    out = contrib[:, 0, :].copy()
    for k in range(1, contrib.shape[1]):
        out = out + contrib[:, k, :]
    return out


def forward_expert_major(x, ids, w, get_expert: Callable[[int], dict], contract: str,
                         return_contrib: bool = False):
    """Routed MoE output for tokens x [T][H] with routes ids [T][K], weights w [T][K].

    Groups the (token, k) slots by expert, runs each expert once on its rows, scatters
    w * y back to the slots and combines. get_expert(e) returns the dict expert_mlp expects.
    """
    x = to_f64(x)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, K = ids.shape
    contrib = None
    for e in np.unique(ids):
        t_idx, k_idx = np.nonzero(ids == e)
        y = expert_mlp(x[t_idx], get_expert(int(e)), contract)
        if contrib is None:
            contrib = np.zeros((T, K, y.shape[1]), dtype=np.float64)
        contrib[t_idx, k_idx, :] = w[t_idx, k_idx][:, None] * y
    out = combine(contrib)
    return (out, contrib) if return_contrib else out


def forward_routed(x, ids, w, get_expert: Callable[[int], dict], contract: str,
                   expert_begin: int = 0, expert_end: int | None = None):
    """Routed MoE output from given routes, restricted to the experts [expert_begin, expert_end).

    Replayed routes are used as recorded instead of being recomputed ([S] §Reinforcement learning
    in Miles); an expert-parallel rank gets explicit ids and weights and computes only its own
    experts ([S] §Fusion Optimizations). Reading: a slot whose expert lies outside the range
    contributes nothing; the remaining contributions w * y are added in k order, starting from 0.
    get_expert(e) takes the global expert id.
    """
    x = to_f64(x)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, K = ids.shape
    hi = np.inf if expert_end is None else expert_end   # None: no upper bound
    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    contrib = np.zeros((T, K, x.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        if not expert_begin <= e < hi:
            continue
        t_idx, k_idx = np.nonzero(ids == e)
        y = expert_mlp(x[t_idx], get_expert(int(e)), contract)
        contrib[t_idx, k_idx, :] = w[t_idx, k_idx][:, None] * y
    for k in range(K):
        out = out + contrib[:, k, :]
    return out


def split_expert(w_gate_up_e, w_down_e, d_ff: int, gate_up_scale=None, down_scale=None) -> dict:
    """Float64 expert dict from one expert's stored tensors (torch or numpy; fp32, bf16 or E4M3
    codes as uint8 when scales are given)."""
    def f64(a):
        try:
            import torch
            if isinstance(a, torch.Tensor):
                if a.dtype == torch.uint8:
                    return e4m3_decode(a.cpu().numpy())
                return a.detach().to("cpu", torch.float64).numpy()
        except ImportError:  # pragma: no cover
            pass
        a = np.asarray(a)
        return e4m3_decode(a) if a.dtype == np.uint8 else a.astype(np.float64)

    gu = f64(w_gate_up_e)
    ex = {"gate": gu[:d_ff], "up": gu[d_ff:], "down": f64(w_down_e)}
    if gate_up_scale is not None:
        s = f64(gate_up_scale)
        ex["gate_scale"], ex["up_scale"], ex["down_scale"] = s[:d_ff], s[d_ff:], f64(down_scale)
    return ex
