"""Hand-worked and printed figures from the pages (tests/golden/), checked against the oracle."""
import os

import numpy as np

from oracle import router

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _parse_cases(path):
    cases, cur = [], None
    for line in open(path, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, _, val = line.partition(":")
        val = val.strip()
        if key == "case":
            cur = {"name": val}
            cases.append(cur)
        else:
            cur[key] = val
    return cases


def _kv(text, E, base):
    v = np.full(E, base)
    for item in text.split():
        k, x = item.split("=")
        v[int(k)] = float(x)
    return v


def test_hand_worked_beam_routing_cases():
    for c in _parse_cases(os.path.join(GOLD, "route_hand_beam.txt")):
        s = _kv(c["s"], 256, float(c["baseline_s"]))[None, :]
        bias = _kv(c["bias"], 256, 0.0)[None, :]
        ids, gscore, kept, mg, me = router.select(s + bias, 8, 4, 8)
        assert list(kept[0]) == [int(v) for v in c["kept_groups"].split()], c["name"]
        assert list(ids[0]) == [int(v) for v in c["ids"].split()], c["name"]
        assert mg[0] == float(c["margin_group"]) and me[0] == float(c["margin_expert"])
        w = router.weights(s, ids, 2.5)
        sel = s[0, ids[0]]
        assert sel.sum() == float(c["sum_s"])
        assert np.allclose(w[0], 2.5 * sel / float(c["sum_s"]), rtol=1e-15)


def test_expert_shape_matches_printed_parameter_counts():
    g = {}
    for line in open(os.path.join(GOLD, "expert_shape.txt"), encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split(":")
            g[k] = float(v)
    per_expert = 3 * g["hidden"] * g["d_ff"]                     # gate, up, down; no biases
    assert abs(per_expert / 1e6 - g["params_per_expert_millions"]) < 0.5
    share = g["moe_layers"] * g["n_experts"] * per_expert / (g["total_params_billions"] * 1e9)
    assert abs(100 * share - g["expert_share_percent"]) < 0.1
    # a fourth matrix or a different d_ff would break the printed figures
    assert abs(4 * g["hidden"] * g["d_ff"] / 1e6 - g["params_per_expert_millions"]) > 5
