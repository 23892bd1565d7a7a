"""Pins of the oracle router against things other than itself: exact rational arithmetic, brute-force
enumeration of group and expert subsets, closed forms and special cases.

Method: [V] §MoE and residual stream; [H] §专家混合; [S] §Dense Layers and Grouped MoE Routing.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import bruteforce
import synthgen
from oracle import router

TINY = dict(n_groups=8, topk_groups=2, topk=4)        # 32 experts, groups of 4
BEAM = dict(n_groups=8, topk_groups=4, topk=8)        # 256 experts, groups of 32
GRID = 2.0 ** -10


def _planted_scores(rng, T, E, ties=True, lo=-0.25, hi=1.25):
    """Selection scores on a 2^-10 grid (so subset sums are exact), with planted ties."""
    ints = rng.integers(int(lo / GRID), int(hi / GRID), size=(T, E))
    if ties:
        for t in range(T):
            n = rng.integers(1, E // 2)
            src = rng.integers(0, E, size=n)
            dst = rng.integers(0, E, size=n)
            ints[t, dst] = ints[t, src]
            if t % 3 == 0:                     # heavy ties: few distinct values
                ints[t] = ints[t] % 5
    return ints


@pytest.mark.parametrize("cfg,E,T", [(TINY, 32, 400), (dict(n_groups=4, topk_groups=2, topk=3), 16, 300),
                                     (dict(n_groups=8, topk_groups=8, topk=4), 16, 100),
                                     (dict(n_groups=1, topk_groups=1, topk=4), 8, 200)])
def test_select_matches_bruteforce(cfg, E, T):
    rng = np.random.default_rng(1)
    ints = _planted_scores(rng, T, E)
    b = ints * GRID
    ids, gscore, kept, mg, me = router.select(b, **cfg)
    for t in range(T):
        kept_bf, chosen_bf, gm_bf, em_bf = bruteforce.select(list(map(int, ints[t])), **cfg)
        assert tuple(sorted(kept[t])) == kept_bf
        assert tuple(sorted(ids[t])) == chosen_bf
        if gm_bf is None:
            assert mg[t] == np.inf
        else:
            assert mg[t] == gm_bf * GRID
        if em_bf is None:
            assert me[t] == np.inf
        else:
            assert me[t] == em_bf * GRID
        # selection order: b descending, ties to the lower id
        order = sorted(ids[t], key=lambda e: (-ints[t][e], e))
        assert list(ids[t]) == order


def test_select_beam_grouping_bruteforce_groups_and_argmax_experts():
    """Beam grouping (8 x 32, keep 4, top 8): groups by brute force over the 70 subsets, experts by
    repeated argmax over the kept groups' members (a different procedure from the oracle's sort)."""
    rng = np.random.default_rng(2)
    ints = _planted_scores(rng, 60, 256)
    b = ints * GRID
    ids, _, kept, _, _ = router.select(b, **BEAM)
    for t in range(60):
        row = list(map(int, ints[t]))
        gsc = bruteforce.group_scores(row, 8)
        _, kept_bf, _ = bruteforce.best_subset(gsc, range(8), 4)
        assert tuple(sorted(kept[t])) == kept_bf
        pool = {e for g in kept_bf for e in range(32 * g, 32 * g + 32)}
        chosen = []
        for _ in range(8):
            best = min(pool, key=lambda e: (-row[e], e))
            chosen.append(best)
            pool.remove(best)
        assert list(ids[t]) == chosen


def test_negative_scores_are_excluded_not_zeroed():
    """Kept groups hold negative b; experts of dropped groups with b = 0 must not be chosen."""
    E = 32
    b = np.zeros((1, E))
    b[0, 0:4] = [-0.5, -0.25, -0.75, -0.125]     # group 0: top-2 sum -0.375
    b[0, 4:8] = [2.0, 1.0, -0.5, -0.5]           # group 1: 3.0
    b[0, 8:] = -1.0                              # all other groups: -2.0
    ids, _, kept, _, _ = router.select(b, **TINY)
    assert sorted(kept[0]) == [0, 1]
    assert list(ids[0]) == [4, 5, 3, 1]


def test_logits_exact_against_fractions():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    w = (0.02 * rng.standard_normal((12, 64))).astype(np.float32)
    z = router.logits(x, w)
    for t in range(5):
        for e in range(12):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(w[e, h])) for h in range(64))
            assert abs(z[t, e] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))


def test_logits_transposed_layout_is_detected():
    """W_r is [E][H]; a transposed read would mix expert and hidden indices."""
    x = np.zeros((1, 4))
    x[0, 1] = 1.0
    w = np.arange(12, dtype=np.float64).reshape(3, 4)     # expert e, hidden h -> 4e + h
    assert list(router.logits(x, w)[0]) == [1.0, 5.0, 9.0]


def test_sigmoid_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 30.0])
    s = router.sigmoid(z)
    assert s[0] == 0.5
    assert abs(s[1] - 0.75) < 1e-15 and abs(s[2] - 0.25) < 1e-15
    assert abs(s[3] - 1.0) < 1e-12


def test_all_ties_special_case():
    """W_r = 0 and bias = 0: every score ties, so the lowest groups and experts win, w = scale/K."""
    d = synthgen.make_inputs("tiny", with_experts=False)
    r = router.route(d["x"], np.zeros((32, 512)), np.zeros(32), routed_scale=2.5, **TINY)
    assert np.all(r.kept_groups == [0, 1])
    assert np.all(r.ids == [0, 1, 2, 3])
    assert np.all(r.weights == 2.5 / 4)
    assert np.all(r.margin == 0.0)


def test_single_group_is_plain_topk():
    rng = np.random.default_rng(4)
    b = rng.standard_normal((50, 32))              # distinct values
    ids, *_ = router.select(b, n_groups=1, topk_groups=1, topk=5)
    ref = np.argsort(-b, axis=1)[:, :5]
    assert np.array_equal(ids, ref)


def test_topk_one_weight_is_scale():
    d = synthgen.make_inputs("tiny", with_experts=False)
    r = router.route(d["x"], d["w_router"], d["bias"], n_groups=8, topk_groups=2, topk=1,
                     routed_scale=2.5)
    assert np.all(r.weights == 2.5)


def test_weights_invariants_and_bias_independence():
    d = synthgen.make_inputs("tiny", with_experts=False)
    r = router.route_cfg(d)
    assert np.allclose(r.weights.sum(axis=1), 2.5, rtol=0, atol=1e-12)
    s_sel = np.take_along_axis(r.s, r.ids, axis=1)
    assert np.allclose(r.weights[:, 0:1] / r.weights, s_sel[:, 0:1] / s_sel, rtol=1e-13)
    # same ids, different bias -> same weights (the bias only chooses)
    w2 = router.weights(r.s, r.ids, 2.5)
    assert np.array_equal(w2, r.weights)
    # ids lie in the kept groups, are distinct and in range
    gs = 32 // 8
    for t in range(d["T"]):
        assert len(set(r.ids[t])) == 4
        assert set(r.ids[t] // gs) <= set(r.kept_groups[t])


def test_bias_changes_choice_only():
    """A large bias on one expert forces it in; its weight still uses the unbiased score."""
    d = synthgen.make_inputs("tiny", with_experts=False)
    bias = np.zeros(32)
    bias[13] = 10.0
    r = router.route(d["x"], d["w_router"], bias, routed_scale=2.5, **TINY)
    assert np.all(r.ids[:, 0] == 13)
    s_sel = np.take_along_axis(r.s, r.ids, axis=1)
    assert np.allclose(r.weights, 2.5 * s_sel / s_sel.sum(axis=1, keepdims=True), rtol=1e-14)
