"""Pins of the boundary oracle (post RMSNorm -> depth-scaled residual -> next RMSNorm): a hand-worked
example, closed forms and invariants ([V] §MoE and residual stream; [S] §Sandwich Normalization and
Depth-Scaled Residuals)."""
import os

import numpy as np
import pytest

from oracle import boundary, codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "boundary_hand.txt")


def _golden():
    vals = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        vals[k] = np.array([float(t) for t in v])
    return vals


def test_hand_worked_example():
    g = _golden()
    h_out, x_next, parts = boundary.boundary(g["y"][None], g["h"][None], g["gamma_post"],
                                             g["gamma_next"], int(g["n"][0]), 0.0,
                                             return_parts=True)
    np.testing.assert_array_equal(parts["p"][0], g["p"])
    np.testing.assert_array_equal(parts["a"][0], g["a"])
    np.testing.assert_array_equal(h_out[0], g["h_out"])
    np.testing.assert_array_equal(x_next[0], g["x_next"])


def test_first_add_keeps_only_the_branch():
    """n = 1 (the add after the embedding): alpha = 0, beta = 1, so h' = p whatever h holds."""
    rng = np.random.default_rng(1)
    y = codecs.bf16_round(rng.standard_normal((5, 64)))
    h = codecs.bf16_round(rng.standard_normal((5, 64)) * 100)
    gp = 1 + rng.uniform(-0.2, 0.2, 64)
    h_out, _, parts = boundary.boundary(y, h, gp, np.ones(64), 1, 1e-6, return_parts=True)
    np.testing.assert_array_equal(h_out, parts["p"])
    assert boundary.residual_coefficients(1) == (0.0, 1.0)


def test_coefficients_keep_unit_scale():
    """alpha^2 + beta^2 = 1 for every n, and after n adds each term carries weight 1/sqrt(n)."""
    for n in range(1, 105):
        a, b = boundary.residual_coefficients(n)
        assert abs(a * a + b * b - 1.0) < 1e-15
    w = [1.0]                       # weights of the embedding and branch outputs in the stream
    for n in range(2, 105):
        a, b = boundary.residual_coefficients(n)
        w = [x * a for x in w] + [b]
    assert np.allclose(w, 1 / np.sqrt(104), rtol=1e-12)


def test_norm_is_scale_invariant_and_unit_rms():
    """RMSNorm with eps = 0: scaling y by a power of two leaves p unchanged; a constant row
    normalises to +-1; with gamma = 1 the normalised row has unit RMS."""
    rng = np.random.default_rng(2)
    y = codecs.bf16_round(rng.standard_normal((4, 128)))
    h = codecs.bf16_round(rng.standard_normal((4, 128)))
    ones = np.ones(128)
    _, _, p1 = boundary.boundary(y, h, ones, ones, 3, 0.0, return_parts=True)
    _, _, p2 = boundary.boundary(8 * y, h, ones, ones, 3, 0.0, return_parts=True)
    np.testing.assert_array_equal(p1["p"], p2["p"])
    c = np.full((1, 128), -3.0)
    _, _, pc = boundary.boundary(c, h[:1], ones, ones, 2, 0.0, return_parts=True)
    np.testing.assert_array_equal(pc["p"], -np.ones((1, 128)))
    r = boundary.rmsnorm(y, ones, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=1)), 1.0, rtol=1e-12)


def test_gamma_on_the_right_axis_and_eps_enters_the_root():
    y = np.array([[1.0, 1.0, 1.0, 1.0]])
    g = np.array([1.0, 2.0, 3.0, 4.0])
    np.testing.assert_allclose(boundary.rmsnorm(y, g, 0.0)[0], g)
    np.testing.assert_allclose(boundary.rmsnorm(y, np.ones(4), 3.0)[0], 0.5)   # 1/sqrt(1+3)
