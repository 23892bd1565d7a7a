"""Brute-force reference for group-limited top-k selection (tests only).

Formulation independent of the oracle's sort-based one: among all Gk-subsets of groups, take the
one with the largest total group score; among all K-subsets of the kept groups' members, take the
one with the largest total selection score. Ties between subsets go to the lexicographically
smallest sorted index tuple. Scores are given as exact integers (multiples of a grid step), so
every comparison is exact. The top-2 group score is found by scanning all member pairs.
"""
from itertools import combinations


def group_scores(b_int, n_groups):
    E = len(b_int)
    gs = E // n_groups
    scores = []
    for g in range(n_groups):
        mem = b_int[g * gs:(g + 1) * gs]
        if gs == 1:
            scores.append(mem[0])
        else:
            scores.append(max(mem[i] + mem[j] for i, j in combinations(range(gs), 2)))
    return scores


def best_subset(values, idx, k):
    """(best sum, best tuple, second-best sum) over k-subsets of idx, ties -> smallest tuple."""
    best = None
    second = None
    for combo in combinations(sorted(idx), k):
        s = sum(values[i] for i in combo)
        if best is None or s > best[0]:
            if best is not None:
                second = best[0] if second is None else max(second, best[0])
            best = (s, combo)
        else:
            second = s if second is None else max(second, s)
    return best[0], best[1], second


def select(b_int, n_groups, topk_groups, topk):
    """Returns (kept group tuple, chosen expert tuple, group margin, expert margin) in grid units."""
    E = len(b_int)
    gs = E // n_groups
    gsc = group_scores(b_int, n_groups)
    _, kept, g_second = best_subset(gsc, range(n_groups), topk_groups)
    g_best = sum(gsc[g] for g in kept)
    cand = [e for g in kept for e in range(g * gs, (g + 1) * gs)]
    e_best, chosen, e_second = best_subset(b_int, cand, topk)
    gm = None if g_second is None else g_best - g_second
    em = None if e_second is None else e_best - e_second
    return kept, chosen, gm, em
