"""Pins of the oracle's expert MLP, rounding contracts and combine against closed forms.

Method: SwiGLU experts without biases, weighted combine with no shared expert ([H] §专家混合;
[V] §MoE and residual stream); bf16 rounding points of [S] §BF16 MoE Kernel Optimization.
"""
import math

import numpy as np
import pytest
import torch

import synthgen
from oracle import codecs, experts, router

H, F, E = 8, 4, 4


def _perm(n):
    return (3 * n + 1) % F


def _selector_experts(c):
    """Expert e: gate row f picks x[1+f]; up row f is c[e] * x[0]; down row n picks h[perm(n)]
    with factor (e+1). With x[0] = 1:  y_e[n] = (e+1) * c[e] * silu(x[1+perm(n)])."""
    ex = {}
    for e in range(E):
        gate = np.zeros((F, H))
        up = np.zeros((F, H))
        down = np.zeros((H, F))
        for f in range(F):
            gate[f, 1 + f] = 1.0
            up[f, 0] = c[e]
        for n in range(H):
            down[n, _perm(n)] = e + 1.0
        ex[e] = {"gate": gate, "up": up, "down": down}
    return ex


def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_selector_experts_fp32_closed_form():
    rng = np.random.default_rng(8)
    c = [0.5, -1.25, 2.0, 0.75]
    ex = _selector_experts(c)
    T, K = 6, 2
    x = rng.standard_normal((T, H))
    x[:, 0] = 1.0
    ids = np.array([[0, 1], [3, 2], [1, 3], [2, 0], [0, 3], [1, 2]])
    w = rng.uniform(0.1, 2.0, size=(T, K))
    out = experts.forward_expert_major(x, ids, w, lambda e: ex[e], "fp32")
    for t in range(T):
        for n in range(H):
            want = sum(w[t][k] * (ids[t][k] + 1) * c[ids[t][k]] * _silu(x[t][1 + _perm(n)])
                       for k in range(K))
            assert abs(out[t][n] - want) <= 1e-14 * max(1.0, abs(want))


def _bf16(v):
    """bf16 RNE of a float64 value by a route independent of the oracle: float64 -> float32 via
    numpy, then torch's fp32 -> bf16 cast, used only where the first step cannot double-round."""
    f = np.float32(v)
    lo = torch.tensor(float(f)).to(torch.bfloat16).item()
    # reject values whose fp32 rounding lands exactly on a bf16 midpoint (double rounding risk)
    bits = np.array([f], dtype=np.float32).view(np.uint32)[0]
    assert (bits & 0xFFFF) != 0x8000 or float(f) == v
    return lo


def test_selector_experts_bf16_rounding_points():
    """g, u, h rounded to bf16; weights applied to y un-rounded; combine un-rounded."""
    c = [0.5, -1.25, 2.0, 0.75]                    # bf16-exact up factors
    ex = _selector_experts(c)
    rng = np.random.default_rng(9)
    T, K = 5, 2
    x = torch.from_numpy(rng.standard_normal((T, H))).to(torch.bfloat16).double().numpy()
    x[:, 0] = 1.0
    ids = np.array([[0, 1], [3, 2], [1, 3], [2, 0], [0, 3]])
    w = rng.uniform(0.1, 2.0, size=(T, K))
    out = experts.forward_expert_major(x, ids, w, lambda e: ex[e], "bf16")
    for t in range(T):
        for n in range(H):
            want = 0.0
            for k in range(K):
                e = ids[t][k]
                g = x[t][1 + _perm(n)]                   # already bf16
                h = _bf16(_silu(g) * c[e])
                want += w[t][k] * (e + 1) * h
            assert abs(out[t][n] - want) <= 1e-14 * max(1.0, abs(want))
    # the rounding points matter: the fp32 contract differs
    out32 = experts.forward_expert_major(x, ids, w, lambda e: ex[e], "fp32")
    assert np.abs(out32 - out).max() > 1e-4


def test_gate_up_order_and_split():
    """split_expert takes gate = rows [0, F), up = rows [F, 2F); swapping them changes the result."""
    rng = np.random.default_rng(10)
    gu = rng.standard_normal((2 * F, H))
    dn = rng.standard_normal((H, F))
    ex = experts.split_expert(gu, dn, F)
    assert np.array_equal(ex["gate"], gu[:F]) and np.array_equal(ex["up"], gu[F:])
    x = rng.standard_normal((3, H))
    y = experts.expert_mlp(x, ex, "fp32")
    g, u = x @ gu[:F].T, x @ gu[F:].T
    want = np.array([[sum(dn[n, f] * _silu(g[t, f]) * u[t, f] for f in range(F)) for n in range(H)]
                     for t in range(3)])
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)
    swapped = experts.expert_mlp(x, {"gate": ex["up"], "up": ex["gate"], "down": dn}, "fp32")
    assert not np.allclose(y, swapped)


@pytest.mark.parametrize("contract", ["fp32", "bf16"])
def test_identical_experts_closed_form(contract):
    """If all experts are the same, out = scale * MLP(x) whatever the routing."""
    d = synthgen.make_inputs("tiny", experts=[5])
    sh = d["workload"].shape
    ex = experts.split_expert(d["w_gate_up_e"][5], d["w_down_e"][5], sh.d_ff)
    r = router.route_cfg(d)
    out = experts.forward_expert_major(d["x"], r.ids, r.weights, lambda e: ex, contract)
    mlp = experts.expert_mlp(router.to_f64(d["x"]), ex, contract)
    assert np.allclose(out, 2.5 * mlp, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance():
    d = synthgen.make_inputs("tiny")
    sh = d["workload"].shape
    get = lambda e: experts.split_expert(d["w_gate_up"][e], d["w_down"][e], sh.d_ff)  # noqa: E731
    r = router.route_cfg(d)
    out = experts.forward_expert_major(d["x"], r.ids, r.weights, get, "bf16")
    perm = np.random.default_rng(11).permutation(d["T"])
    xp = d["x"][torch.from_numpy(perm)]
    rp = router.route(xp, d["w_router"], d["bias"], 8, 2, 4, 2.5)
    assert np.array_equal(rp.ids, r.ids[perm])
    outp = experts.forward_expert_major(xp, rp.ids, rp.weights, get, "bf16")
    assert np.allclose(outp, out[perm], rtol=1e-12, atol=1e-14)


def test_fp8_contract_exact_case():
    """Power-of-two scales and E4M3-exact values: every fp8 step is exact, so the output has a
    closed form; per-token and per-channel scales must land on the right axes."""
    F8, H8 = 2, 4
    # token rows: amax 448 * 2^-4 = 28 -> scale 2^-4, codes exact
    x = np.array([[28.0, 1.0, -2.0, 0.5], [-28.0, 0.25, 3.0, 1.0]])
    gate_codes = np.zeros((F8, H8)); gate_codes[0, 1] = 1.0; gate_codes[1, 2] = 1.0
    up_codes = np.zeros((F8, H8)); up_codes[0, 0] = 1.0; up_codes[1, 0] = 0.5
    down_codes = np.zeros((H8, F8)); down_codes[:, 0] = 1.0; down_codes[1, 1] = 2.0
    ex = {"gate": gate_codes, "up": up_codes, "down": down_codes,
          "gate_scale": np.array([0.5, 2.0]), "up_scale": np.array([0.25, 1.0]),
          "down_scale": np.array([1.0, 2.0, 4.0, 0.5])}
    y = experts.expert_mlp(x, ex, "fp8")
    for t in range(2):
        g = [0.5 * x[t][1], 2.0 * x[t][2]]          # s_x * codes cancel (x is on the grid)
        u = [0.25 * x[t][0], 0.5 * x[t][0]]
        h = [_bf16(_silu(g[f]) * u[f]) for f in range(F8)]
        amax = max(abs(v) for v in h)
        qh, sh = codecs.quant_rows_fp8(np.array([h], dtype=np.float32))
        hd = codecs.e4m3_decode(qh[0]) * float(sh[0])
        assert abs(max(abs(v) for v in hd) - amax) <= amax * 2 ** -4
        for n in range(H8):
            want = ex["down_scale"][n] * sum(down_codes[n, f] * hd[f] for f in range(F8))
            assert abs(y[t][n] - want) <= 1e-14 * max(1.0, abs(want))


def test_routed_range_closed_form():
    """Given routes over a range of experts ([S] §Fusion Optimizations, §Reinforcement learning in
    Miles): only slots routed into [begin, end) contribute, with their weights as given; ids
    outside [0, E) never contribute."""
    rng = np.random.default_rng(11)
    c = [0.5, -1.25, 2.0, 0.75]
    ex = _selector_experts(c)
    T, K = 7, 3
    x = rng.standard_normal((T, H))
    x[:, 0] = 1.0
    ids = np.array([[0, 1, 2], [3, 2, 1], [1, 3, 0], [2, 0, 3], [0, 3, -1], [1, 2, 9], [3, 0, 1]])
    w = rng.uniform(-1.0, 2.0, size=(T, K))   # arbitrary: no renormalisation is implied
    for begin, end in [(0, 4), (1, 3), (2, 3), (0, 1), (3, 4), (2, 2)]:
        out = experts.forward_routed(x, ids, w, lambda e: ex[e], "fp32", begin, end)
        for t in range(T):
            for n in range(H):
                want = sum(w[t][k] * (ids[t][k] + 1) * c[ids[t][k]] * _silu(x[t][1 + _perm(n)])
                           for k in range(K) if begin <= ids[t][k] < end)
                assert abs(out[t][n] - want) <= 1e-14 * max(1.0, abs(want)), (begin, end, t, n)


@pytest.mark.parametrize("contract", ["fp32", "bf16"])
def test_routed_partition_sums_to_forward(contract):
    """Outputs over a partition of the experts add up to the full routed MoE output; the full range
    reproduces it exactly."""
    rng = np.random.default_rng(12)
    ex = {e: {"gate": rng.standard_normal((F, H)) * 0.3, "up": rng.standard_normal((F, H)) * 0.3,
              "down": rng.standard_normal((H, F)) * 0.3} for e in range(E)}
    T, K = 9, 2
    x = rng.standard_normal((T, H))
    ids = np.array([rng.choice(E, size=K, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.5, size=(T, K))
    full = experts.forward_expert_major(x, ids, w, lambda e: ex[e], contract)
    np.testing.assert_array_equal(
        experts.forward_routed(x, ids, w, lambda e: ex[e], contract, 0, E), full)
    parts = sum(experts.forward_routed(x, ids, w, lambda e: ex[e], contract, b, e)
                for b, e in [(0, 1), (1, 3), (3, 4)])
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12)
