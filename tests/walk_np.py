"""A second, independent implementation of the selection walk for tiny inputs.

Written separately from the C oracle, in numpy with scipy's ``logsumexp``, straight from
the definitions ("Block Sparse Attention with Log-Linear Complexity": agihunt.info pyramid
and LSE/forced-block paragraphs, rcap.io top-down walk paragraph) and the readings listed
in the design notes.  It shares no code with the oracle; tests compare the two.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def level_sizes(N, C, K, g):
    sizes = [N, math.ceil(N / C)]
    while sizes[-1] > g * K:
        sizes.append(math.ceil(sizes[-1] / g))
    return sizes  # sizes[l] for l = 0..L


def pyramid(keys: np.ndarray, C: int, K: int, g: int):
    """keys [N, d] float64 -> list of level arrays, levels[l] = [n_l, d] for l >= 1."""
    N = keys.shape[0]
    sizes = level_sizes(N, C, K, g)
    levels = [keys]
    levels.append(np.stack([keys[j * C: min(j * C + C, N)].mean(axis=0) for j in range(sizes[1])]))
    for l in range(2, len(sizes)):
        prev = levels[l - 1]
        levels.append(np.stack([prev[j * g: min(j * g + g, sizes[l - 1])].mean(axis=0)
                                for j in range(sizes[l])]))
    return levels


def select_one(qrows: np.ndarray, keys: np.ndarray, i: int, C: int, K: int, g: int, s: float, scorer: int = 0):
    """qrows [G, d], keys [N, d] (float64).  Returns (idx list, score list) of length K.

    scorer 0 routes by the LSE over a node's visible children, 1 by log m + their mean
    (PISA-1), 2 by that plus half their population variance (PISA-2).
    """
    N = keys.shape[0]
    levels = pyramid(keys, C, K, g)
    L = len(levels) - 1
    b = i // C

    def first_leaf(l, j):
        return j * g ** (l - 1)

    def children(l, j):
        return [c for c in range(j * g, min(j * g + g, len(levels[l - 1]))) if first_leaf(l - 1, c) <= b]

    def route_score(l, j):
        kids = children(l, j)
        dots = s * (qrows @ levels[l - 1][kids].T)  # [G, |kids|]
        if scorer == 0:
            return float(logsumexp(dots, axis=1).sum())
        per_head = math.log(len(kids)) + dots.mean(axis=1)
        if scorer == 2:
            per_head = per_head + dots.var(axis=1) / 2
        return float(per_head.sum())

    def leaf_score(j):
        hi = min(j * C + C, N, i + 1)
        dots = s * (qrows @ keys[j * C: hi].T)
        return float(logsumexp(dots, axis=1).sum())

    def top(cands, score_fn, m):
        ranked = sorted(cands, key=lambda j: (-score_fn(j), j))
        return ranked[:m]

    if L == 1:
        cand = list(range(b + 1))
    else:
        cand = [j for j in range(len(levels[L])) if first_leaf(L, j) <= b]
        for l in range(L, 1, -1):
            kept = top(cand, lambda j, l=l: route_score(l, j), K)
            cand = [c for j in kept for c in children(l, j)]
    forced = sorted({0, b - 1, b} & set(range(b + 1)))
    rest = [j for j in cand if j not in forced]
    chosen = sorted(forced + top(rest, leaf_score, K - len(forced)))
    idx = chosen + [-1] * (K - len(chosen))
    sc = [leaf_score(j) for j in chosen] + [-math.inf] * (K - len(chosen))
    return idx, sc
