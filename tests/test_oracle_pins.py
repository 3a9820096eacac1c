"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Every pin here checks the oracle against something other than itself: exact identities,
closed forms derived by hand (``tests/golden``), library routines (scipy's logsumexp,
numpy means), brute force on tiny inputs, and invariants the definitions imply.
Citations: "Block Sparse Attention with Log-Linear Complexity", agihunt.info summary
(pyramid paragraph; LSE and forced-block paragraph; kernels/GQA paragraph) and rcap.io
explainer (tree/pooling paragraph; top-down walk paragraph with the g*K bound; scoring
paragraph with the Jensen remark; the paragraph on Appendix A's sandwich).
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from block_selection_pyramid_amd import synth

from walk_np import select_one

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32, BF16 = oracle.F32, oracle.BF16


def rng_arrays(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


# --------------------------------------------------------------- LSE identities

def test_lse_identities():
    r = np.random.default_rng(0)
    for n in [1, 2, 3, 17, 64]:
        x = r.standard_normal(n) * 5
        c = float(r.standard_normal() * 10)
        assert oracle.lse([x[0]]) == x[0]
        assert math.isclose(oracle.lse(x + c), oracle.lse(x) + c, rel_tol=0, abs_tol=1e-12)
        a, b = x[: n // 2], x[n // 2:]
        if len(a) and len(b):
            assert math.isclose(oracle.lse(x), oracle.lse([oracle.lse(a), oracle.lse(b)]), abs_tol=1e-12)
        assert math.isclose(oracle.lse(np.full(n, x[0])), x[0] + math.log(n), abs_tol=1e-12)
        assert x.max() <= oracle.lse(x) <= x.max() + math.log(n) + 1e-12
        # library routine
        assert math.isclose(oracle.lse(x), float(logsumexp(x)), abs_tol=1e-12)
    assert oracle.lse([-math.inf, 1.0]) == 1.0
    assert oracle.lse([-math.inf]) == -math.inf
    assert oracle.lse([1000.0, 1000.0]) == pytest.approx(1000.0 + math.log(2), abs=1e-12)


# ----------------------------------------------------------------- level table

@pytest.mark.parametrize("N,K,expect", [
    (1024, 4, [16, 8]),
    (4096, 8, [64, 32, 16]),
    (16384, 32, [256, 128, 64]),
    (65536, 8, [1024, 512, 256, 128, 64, 32, 16]),
    (131072, 8, [2048, 1024, 512, 256, 128, 64, 32, 16]),
    (262144, 8, [4096, 2048, 1024, 512, 256, 128, 64, 32, 16]),
])
def test_level_tables(N, K, expect):
    assert oracle.levels(N, 64, K, 2)[1:] == expect


def test_level_count_closed_form():
    # L = 1 + ceil(log_g(n_1 / (g K))) once n_1 > g K (pyramid paragraph: O(log N) levels)
    for e in range(10, 19):
        N = 2 ** e
        for K in (4, 8, 32):
            n1 = N // 64
            L = len(oracle.levels(N, 64, K, 2)) - 1
            want = 1 if n1 <= 2 * K else 1 + math.ceil(math.log2(n1 / (2 * K)))
            assert L == want
    assert oracle.levels(1000, 64, 8, 2)[1:] == [16]
    assert oracle.levels(5000, 64, 8, 3)[1:] == [79, 27, 9]


# --------------------------------------------------------------------- pyramid

def test_pyramid_is_direct_mean_on_full_trees():
    p = oracle.Problem(1, 64 * 64, 1, 2, 16, 64, 4, 2, dtype=F32)
    k = rng_arrays(1, (1, 2, p.seq_len, 16))
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(p.seq_len, 64, 4, 2)
    off = 0
    for l in range(1, len(sizes)):
        span = 64 * 2 ** (l - 1)
        for h in range(2):
            direct = k[0, h].astype(np.float64).reshape(sizes[l], span, 16).mean(axis=1)
            np.testing.assert_allclose(pyr[0, h, off: off + sizes[l]], direct, rtol=0, atol=1e-12)
        off += sizes[l]
    assert off == pyr.shape[2]


def test_pyramid_ragged_tail_and_odd_levels():
    # N = 5*64 + 7: the last leaf averages its 7 present keys; odd counts leave
    # single-child nodes whose mean is that child.
    N, K, g = 5 * 64 + 7, 3, 2
    p = oracle.Problem(1, N, 1, 1, 4, 64, K, g, dtype=F32)
    k = rng_arrays(2, (1, 1, N, 4))
    pyr = oracle.build_pyramid(p, k)[0, 0]
    sizes = oracle.levels(N, 64, K, g)
    assert sizes[1:] == [6]  # n1 = 6 <= g*K = 6 -> L = 1
    kd = k[0, 0].astype(np.float64)
    np.testing.assert_allclose(pyr[5], kd[320:327].mean(axis=0), atol=1e-12)
    p2 = oracle.Problem(1, N, 1, 1, 4, 64, 3, 2, dtype=F32)
    N2 = 13 * 64 + 1  # n1 = 14 -> 7 -> L=2 with K=3 (gK = 6 < 7?) -> n = [14, 7, 4]
    p2 = oracle.Problem(1, N2, 1, 1, 4, 64, 3, 2, dtype=F32)
    k2 = rng_arrays(3, (1, 1, N2, 4))
    pyr2 = oracle.build_pyramid(p2, k2)[0, 0]
    s2 = oracle.levels(N2, 64, 3, 2)
    assert s2[1:] == [14, 7, 4]
    kd2 = k2[0, 0].astype(np.float64)
    np.testing.assert_allclose(pyr2[13], kd2[832:833].mean(axis=0), atol=1e-12)
    lv2 = pyr2[14:21]
    np.testing.assert_allclose(lv2[6], (pyr2[12] + pyr2[13]) / 2, atol=1e-12)
    lv3 = pyr2[21:25]
    np.testing.assert_allclose(lv3[3], lv2[6], atol=1e-12)  # single child
    np.testing.assert_allclose(lv3[0], kd2[0:256].mean(axis=0), atol=1e-12)


def test_bf16_inputs_are_read_exactly():
    x = rng_arrays(4, (1, 1, 128, 8))
    bits = synth.to_bf16_bits(x)
    vals = synth.bf16_bits_to_f32(bits).astype(np.float64)
    p = oracle.Problem(1, 128, 1, 1, 8, 64, 3, 2, dtype=BF16)
    pyr = oracle.build_pyramid(p, bits)
    np.testing.assert_allclose(pyr[0, 0, 0], vals[0, 0, :64].mean(axis=0), atol=1e-15)
    # bf16 rounding is nearest-even on the float value
    assert np.all(np.abs(vals - x) <= np.abs(x) * 2.0 ** -8 + 1e-30)


# ---------------------------------------------------------- golden hand cases

def _golden_inputs(g):
    P = g["problem"]
    p = oracle.Problem(P["batch"], P["seq_len"], P["n_q_heads"], P["n_kv_heads"], P["head_dim"], P["block"],
                       P["top_k"], P["branch"], scale=P.get("scale", 0.0), dtype=F32)
    return p


def test_golden_zero_keys():
    g = json.load(open(os.path.join(GOLDEN, "zero_keys.json")))
    p = _golden_inputs(g)
    assert oracle.levels(p.seq_len, p.block, p.top_k, p.branch) == g["levels"]
    q = rng_arrays(5, (1, p.n_q_heads, p.seq_len, p.head_dim))
    k = np.zeros((1, 1, p.seq_len, p.head_dim), dtype=np.float32)
    rows = [c["i"] for c in g["cases"]]
    idx, sc = oracle.select(p, q, k, rows=rows)
    for t, c in enumerate(g["cases"]):
        assert idx[t].tolist() == c["idx"], c
        want = [p.group * math.log(n) if n else -math.inf for n in c["keys_seen"]]
        for a, b in zip(sc[t], want):
            assert (a == b) if math.isinf(b) else abs(a - b) < 1e-12


def test_golden_monotone_keys_equal_brute_force():
    g = json.load(open(os.path.join(GOLDEN, "monotone_keys.json")))
    p = _golden_inputs(g)
    N, C, d = p.seq_len, p.block, p.head_dim
    q = np.zeros((1, p.n_q_heads, N, d), dtype=np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d), dtype=np.float32)
    k[0, 0, :, 0] = 8.0 * (np.arange(N) // C)
    rows = [c["i"] for c in g["cases"]]
    idx, sc = oracle.select(p, q, k, rows=rows)
    for t, c in enumerate(g["cases"]):
        assert idx[t].tolist() == c["idx"], (c, idx[t])
        for j, n, s in zip(c["idx"], c["keys_seen"], sc[t]):
            if j < 0:
                assert s == -math.inf
            else:
                assert abs(s - p.group * (2 * j + math.log(n))) < 1e-9
    # and for every row: {0} u [max(1, b-K+2), b]
    allidx, _ = oracle.select(p, q, k)
    for i in range(0, N, 37):
        b = i // C
        want = sorted({0} | set(range(max(1, b - p.top_k + 2), b + 1)))
        assert allidx[i].tolist() == want + [-1] * (p.top_k - len(want))


# ---------------------------------------------------------- leaf and causal

def test_leaf_score_closed_forms():
    p = oracle.Problem(1, 1024, 4, 2, 32, 64, 4, 2, dtype=F32)
    q = rng_arrays(6, (1, 4, 1024, 32))
    k = rng_arrays(7, (1, 2, 1024, 32))
    s = p.s
    for h in range(2):
        for b in (0, 3, 15):
            i = 64 * b
            row = h * 1024 + i
            tot, ph = oracle.leaf_score(p, q, k, row, b)
            want = [s * float(q[0, h * 2 + r, i].astype(np.float64) @ k[0, h, i].astype(np.float64))
                    for r in range(2)]
            np.testing.assert_allclose(ph, want, atol=1e-12)
            assert abs(tot - sum(want)) < 1e-12
            i2 = i + 1
            _, ph2 = oracle.leaf_score(p, q, k, h * 1024 + i2, b)
            for r in range(2):
                x = [s * float(q[0, h * 2 + r, i2].astype(np.float64) @ k[0, h, t].astype(np.float64))
                     for t in (i, i + 1)]
                assert abs(ph2[r] - float(logsumexp(x))) < 1e-12


def _prefill(seed, N, Hq, Hkv, d, K, dtype=F32, g=2, needles=2, B=1):
    w = synth.custom(batch=B, seq_len=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, top_k=K, branch=g,
                     dtype=dtype, seed=seed, needles=needles)
    q, k, _ = synth.make_inputs(w)
    p = oracle.Problem(B, N, Hq, Hkv, d, 64, K, g, dtype=dtype)
    return p, q, k


@pytest.mark.parametrize("N,K,G", [(1024, 4, 1), (3000, 8, 2), (4096 + 37, 3, 4), (777, 5, 1)])
def test_selection_invariants(N, K, G):
    p, q, k = _prefill(10 + N, N, 2 * G, 2, 16, K, B=2)
    idx, sc = oracle.select(p, q, k)
    idx = idx.reshape(2, 2, N, K)
    sc = sc.reshape(2, 2, N, K)
    for i in range(N):
        b = i // 64
        for bb in range(2):
            for h in range(2):
                row = idx[bb, h, i]
                n = int((row >= 0).sum())
                assert n == min(K, b + 1)
                sel = row[:n]
                assert np.all(np.diff(sel) > 0) and sel.max() <= b and sel.min() >= 0
                assert np.all(row[n:] == -1) and np.all(np.isneginf(sc[bb, h, i, n:]))
                for f in {0, b - 1, b}:
                    if f >= 0:
                        assert f in sel


# ------------------------------------------------------ reduces to brute force

def brute_force(p, q, k, row):
    """F u TopK_{K-|F|} over every causal leaf block by raw-key LSE (numpy/scipy)."""
    N, C, G = p.seq_len, p.block, p.group
    bh, i = divmod(row, N)
    b, h = divmod(bh, p.n_kv_heads)
    qr = q[b, h * G:(h + 1) * G, i].astype(np.float64)
    kk = k[b, h].astype(np.float64)
    bq = i // C
    scores = {}
    for j in range(bq + 1):
        hi = min(j * C + C, N, i + 1)
        scores[j] = float(logsumexp(p.s * (qr @ kk[j * C:hi].T), axis=1).sum())
    F = sorted({0, bq - 1, bq} & set(range(bq + 1)))
    rest = sorted([j for j in scores if j not in F], key=lambda j: (-scores[j], j))
    sel = sorted(F + rest[: p.top_k - len(F)])
    return sel, [scores[j] for j in sel]


def test_L1_regime_equals_brute_force():
    # n_1 = 16 <= g*K = 16: the walk starts at the leaf level and scores every causal block
    p, q, k = _prefill(21, 1024, 2, 1, 32, 8)
    assert len(oracle.levels(1024, 64, 8, 2)) - 1 == 1
    idx, sc = oracle.select(p, q, k)
    for i in range(0, 1024, 7):
        sel, s = brute_force(p, q, k, i)
        assert idx[i, : len(sel)].tolist() == sel
        np.testing.assert_allclose(sc[i, : len(sel)], s, atol=1e-9)


def test_K_at_least_blocks_selects_every_causal_block():
    p, q, k = _prefill(22, 1024, 1, 1, 64, 16)
    idx, _ = oracle.select(p, q, k)
    for i in range(1024):
        b = i // 64
        assert idx[i, : b + 1].tolist() == list(range(b + 1))
        assert np.all(idx[i, b + 1:] == -1)


# ------------------------------------------------- Jensen sandwich (Appendix A)

def test_jensen_sandwich_intermediate_scores():
    # log g + s<q, P_l[j]>  <=  S_h(l, j)  <=  LSE over node j's raw keys - log(C g^(l-2))
    N, C, g, K, d = 64 * 64, 64, 2, 4, 16
    p, q, k = _prefill(23, N, 2, 1, d, K)
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(N, C, K, g)
    offs = np.cumsum([0] + sizes[1:])
    kd = k[0, 0].astype(np.float64)
    i = N - 1
    for l in range(2, len(sizes)):
        for j in range(sizes[l]):
            _, ph = oracle.node_score(p, q, pyr, i, l, j)
            node_mean = pyr[0, 0, offs[l - 1] + j]
            span = C * g ** (l - 1)
            raw = kd[j * span:(j + 1) * span]
            for r in range(2):
                qq = q[0, r, i].astype(np.float64)
                lower = math.log(g) + p.s * float(qq @ node_mean)
                upper = float(logsumexp(p.s * (raw @ qq))) - math.log(C * g ** (l - 2))
                assert lower - 1e-9 <= ph[r] <= upper + 1e-9


# ------------------------------------------------------------ O(log N) counts

def test_candidates_bounded_and_work_logarithmic():
    C, K, g, d = 64, 8, 2, 8
    seen = []
    for e in range(11, 20, 2):
        N = 2 ** e
        p, q, k = _prefill(30 + e, N, 1, 1, d, K, needles=0)
        rows = [N - 1, N // 2 + 5, N - 200]
        _, _, st = oracle.select(p, q, k, rows=rows, stats=True)
        L = len(oracle.levels(N, C, K, g)) - 1
        assert np.all(st["max_cand"] <= g * K)
        assert np.all(st["levels"] == L)
        bound = (L - 1) * g * g * K + (g * K + 3) * C
        assert np.all(st["dots"] <= bound)
        brute = (N - 1) // C * C + 1
        if e >= 15:
            assert st["dots"][0] < brute / 4
        seen.append((int(st["dots"][0]), brute))
    # per-query work stays within a constant band while a full scan grows 128x
    work = [w for w, _ in seen]
    assert max(work) / min(work) < 1.6 and seen[-1][1] / seen[0][1] > 100


# ------------------------------------------------------------------- GQA rule

def test_gqa_identical_heads_scale_scores():
    # G identical query heads give the single-head selection, scores times G
    N, d, K = 4096, 16, 8
    p1, q1, k = _prefill(40, N, 1, 1, d, K)
    G = 4
    qG = np.ascontiguousarray(np.repeat(q1, G, axis=1))
    pG = oracle.Problem(1, N, G, 1, d, 64, K, 2, dtype=F32)
    rows = list(range(0, N, 13))
    i1, s1 = oracle.select(p1, q1, k, rows=rows)
    iG, sG = oracle.select(pG, qG, k, rows=rows)
    assert np.array_equal(i1, iG)
    fin = i1 >= 0
    np.testing.assert_allclose(sG[fin], G * s1[fin], rtol=1e-12)


def test_gqa_group_is_sum_of_heads():
    N, d, K = 2048, 16, 8
    p, q, k = _prefill(41, N, 4, 2, d, K)
    pyr = oracle.build_pyramid(p, k)
    for row in (5, N + 700, 2 * N - 1):
        tot, ph = oracle.leaf_score(p, q, k, row, 0)
        assert abs(tot - ph.sum()) < 1e-12
        tot2, ph2 = oracle.node_score(p, q, pyr, row, 2, 0)
        assert abs(tot2 - ph2.sum()) < 1e-12


# ----------------------------------------------------------- decode == prefill

def test_decode_equals_last_prefill_row():
    N, K = 4096 + 11, 8
    p, q, k = _prefill(50, N, 4, 2, 16, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    qdec = np.ascontiguousarray(q[:, :, N - 1, :])
    idd, sd = oracle.select(p, qdec, k, pyr, decode=True)
    rows = [(b * 2 + h) * N + N - 1 for b in range(2) for h in range(2)]
    ip, sp = oracle.select(p, q, k, pyr, rows=rows)
    assert np.array_equal(idd, ip)
    np.testing.assert_array_equal(sd, sp)


# --------------------------------------------------- independent second walk

@pytest.mark.parametrize("N,K,G,g", [(1024, 4, 1, 2), (2048 + 50, 4, 2, 2), (3000, 3, 1, 3)])
def test_matches_independent_numpy_walk(N, K, G, g):
    p, q, k = _prefill(60 + N, N, G, 1, 16, K, g=g)
    pyr = oracle.build_pyramid(p, k)
    rows = list(range(0, N, 29)) + [N - 1]
    idx, sc = oracle.select(p, q, k, pyr, rows=rows)
    kd = k[0, 0].astype(np.float64)
    for t, i in enumerate(rows):
        wi, ws = select_one(q[0, :, i].astype(np.float64), kd, i, 64, K, g, p.s)
        if idx[t].tolist() != wi:
            # only acceptable where the two fp64 orders of summation tie-break differently
            st, _ = oracle.check(p, q, k, pyr, [i], np.array([wi]), np.array([ws], dtype=np.float32),
                                 tau=1e-9, rtol=1e-9)
            assert st[0] == 0, (i, idx[t], wi)
        else:
            np.testing.assert_allclose(sc[t][np.isfinite(sc[t])], np.array(ws)[np.isfinite(ws)], rtol=1e-12)


# --------------------------------------------------------- strong needle found

def test_dominant_needle_is_found():
    # a key aligned to query i with a huge norm dominates every LSE on its path
    N, d, K = 8192, 16, 8
    p, q, k = _prefill(70, N, 1, 1, d, K, needles=0)
    r = np.random.default_rng(3)
    for _ in range(6):
        i = int(r.integers(1000, N))
        pos = int(r.integers(0, i - 200))
        kk = k.copy()
        kk[0, 0, pos] = 4000.0 * q[0, 0, i] / np.linalg.norm(q[0, 0, i])
        idx, _ = oracle.select(p, q, kk, rows=[i])
        assert pos // 64 in idx[0].tolist()


# ------------------------------------------ PISA-1 / PISA-2 routing scorers
# The ablations replace a routing node's per-head LSE over its visible children by the
# first- or second-order truncation of its expansion about the children's mean
# (agihunt.info LSE paragraph; rcap.io scoring-rule paragraph).  The pins below tie the two
# truncations to the oracle's pinned LSE and pyramid, never to a retyped formula.

PISA1, PISA2 = oracle.PISA1, oracle.PISA2


def _visible_children(sizes, l, j, bq, g):
    return [c for c in range(j * g, min(j * g + g, sizes[l - 1])) if c * g ** (l - 2) <= bq]


def _three_scores(p, q, pyr, row, l, j):
    return [oracle.node_score(replace(p, scorer=s), q, pyr, row, l, j)[1] for s in (oracle.LSE, PISA1, PISA2)]


def test_pisa_two_children_log_cosh():
    # two children with dots a, b: LSE - PISA-1 = log cosh((a-b)/2) and
    # PISA-2 - PISA-1 = ((a-b)/2)^2 / 2, so PISA-2 - PISA-1 = acosh(exp(LSE - PISA-1))^2 / 2;
    # one child: all three equal its dot
    N, K, g = 64 * 200 + 9, 4, 2
    p, q, k = _prefill(80, N, 2, 1, 16, K)
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(N, 64, K, g)
    seen = {1: 0, 2: 0}
    for i in (N - 1, 64 * 131 + 5, 64 * 64):
        bq = i // 64
        for l in range(2, len(sizes)):
            for j in range(sizes[l]):
                m = len(_visible_children(sizes, l, j, bq, g))
                if m == 0:
                    continue
                e, a, b = _three_scores(p, q, pyr, i, l, j)
                seen[m] += 1
                if m == 1:
                    np.testing.assert_allclose(a, e, rtol=0, atol=1e-12)
                    np.testing.assert_allclose(b, e, rtol=0, atol=1e-12)
                    continue
                assert np.all(a <= e + 1e-12) and np.all(e <= b + 1e-12)  # log cosh t <= t^2/2
                half_gap = np.arccosh(np.exp(e - a))
                np.testing.assert_allclose(b - a, half_gap ** 2 / 2, rtol=1e-6, atol=1e-10)
    assert seen[1] > 0 and seen[2] > 20


def test_pisa1_of_fully_visible_node_is_parent_mean():
    # when every existing child is visible, the mean of the children's dots is the dot with
    # their mean, which is the parent node itself: PISA-1 = log m + s <q, P_l[j]>
    N, K, g = 64 * 90 + 40, 3, 3  # ragged: the last node of a level may have fewer children
    p, q, k = _prefill(81, N, 2, 1, 16, K, g=g)
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(N, 64, K, g)
    offs = np.cumsum([0] + sizes[1:])
    i = N - 1
    bq = i // 64
    n = 0
    for l in range(2, len(sizes)):
        for j in range(sizes[l]):
            kids = _visible_children(sizes, l, j, bq, g)
            m = min(j * g + g, sizes[l - 1]) - j * g
            if len(kids) != m:
                continue
            _, a = oracle.node_score(replace(p, scorer=PISA1), q, pyr, i, l, j)
            for r in range(2):
                expect = math.log(m) + p.s * float(q[0, r, i].astype(np.float64) @ pyr[0, 0, offs[l - 1] + j])
                assert abs(a[r] - expect) < 1e-10
            n += 1
    assert n > 10


def test_pisa_truncation_orders_in_the_small_scale_limit():
    # with the dots scaled by t -> 0: LSE - PISA-1 = t^2 Var/2 + O(t^3) (halving t quarters
    # it) while LSE - PISA-2 = O(t^3) (halving t divides it by 8, or 16 for two children
    # whose third cumulant vanishes); partially visible nodes (m < g) pin log m, not log g
    N, K, g = 64 * 60 + 17, 3, 3
    p, q, k = _prefill(82, N, 2, 1, 16, K, g=g)
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(N, 64, K, g)
    checked = {2: 0, 3: 0}
    for i in (N - 1, N - 1 - 64 * 4, 64 * 19 + 3):
        bq = i // 64
        for l in range(2, len(sizes)):
            for j in range(sizes[l]):
                m = len(_visible_children(sizes, l, j, bq, g))
                if m < 2:
                    continue
                d1, d2 = [], []
                for t in (2.0 ** -5, 2.0 ** -6):
                    e, a, b = _three_scores(replace(p, scale=p.s * t), q, pyr, i, l, j)
                    d1.append(e - a)
                    d2.append(e - b)
                r1 = d1[0] / d1[1]
                r2 = np.abs(d2[0]) / np.maximum(np.abs(d2[1]), 1e-300)
                assert np.all(np.abs(r1 - 4) < 0.3), (l, j, m, r1)
                assert np.all(r2 > 7) and np.all(np.abs(d2[1]) < 1e-2 * d1[1]), (l, j, m, r2)
                if m == 2:
                    assert np.all(np.abs(r2 - 16) < 2), (l, j, r2)
                checked[m] += 1
    assert checked[2] > 0 and checked[3] > 5


def test_pisa1_below_lse_for_any_branching():
    # Jensen: the mean of the dots never exceeds log mean exp of them
    N, K, g = 64 * 100, 3, 4
    p, q, k = _prefill(83, N, 4, 2, 16, K, g=g)
    pyr = oracle.build_pyramid(p, k)
    sizes = oracle.levels(N, 64, K, g)
    for row in (N - 1, 2 * N - 1, N + 3000):
        bq = (row % N) // 64
        for l in range(2, len(sizes)):
            for j in range(sizes[l]):
                if not _visible_children(sizes, l, j, bq, g):
                    continue
                e, a, b = _three_scores(p, q, pyr, row, l, j)
                assert np.all(a <= e + 1e-12)
                assert np.all(b >= a - 1e-12)  # the variance term is non-negative


def test_pisa_selection_invariants_and_exact_leaf_scores():
    # the scorers only change which leaf candidates survive the routing levels: the result
    # keeps the forced blocks and the K-slot layout, and every reported score is the exact
    # causal leaf LSE of its block
    N, K = 4096 + 37, 6
    p, q, k = _prefill(84, N, 4, 2, 16, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    rows = list(range(0, N, 37)) + [N - 1, 3 * N + 2000, 4 * N - 1]
    base, _ = oracle.select(p, q, k, pyr, rows=rows)
    differs = 0
    for scorer in (PISA1, PISA2):
        ps = replace(p, scorer=scorer)
        idx, sc = oracle.select(ps, q, k, pyr, rows=rows)
        differs += int((idx != base).any(axis=1).sum())
        for t, row in enumerate(rows):
            b = (row % N) // 64
            n = int((idx[t] >= 0).sum())
            assert n == min(K, b + 1)
            sel = idx[t, :n]
            assert np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() <= b
            assert {f for f in (0, b - 1, b) if f >= 0} <= set(sel.tolist())
            for u, j in enumerate(sel):
                assert abs(sc[t, u] - oracle.leaf_score(p, q, k, row, int(j))[0]) < 1e-12
        st, _ = oracle.check(ps, q, k, pyr, rows, idx, sc.astype(np.float32), tau=1e-9, rtol=1e-6)
        assert np.all(st == 0)
    assert differs > 0  # the truncations do change some selections at this size


def test_pisa_scorers_do_not_matter_without_routing_levels():
    # L == 1 (every leaf block fits in g*K): selection is leaf scoring alone
    N, K = 64 * 16, 8
    p, q, k = _prefill(85, N, 2, 1, 16, K)
    assert len(oracle.levels(N, 64, K, 2)) == 2
    i0, s0 = oracle.select(p, q, k)
    for scorer in (PISA1, PISA2):
        i1, s1 = oracle.select(replace(p, scorer=scorer), q, k)
        assert np.array_equal(i0, i1)
        np.testing.assert_array_equal(s0, s1)


@pytest.mark.parametrize("scorer", [PISA1, PISA2])
def test_pisa_decode_equals_last_prefill_row(scorer):
    N, K = 4096 + 11, 8
    p, q, k = _prefill(86, N, 4, 2, 16, K, B=2)
    p = replace(p, scorer=scorer)
    pyr = oracle.build_pyramid(p, k)
    qdec = np.ascontiguousarray(q[:, :, N - 1, :])
    idd, sd = oracle.select(p, qdec, k, pyr, decode=True)
    rows = [(b * 2 + h) * N + N - 1 for b in range(2) for h in range(2)]
    ip, sp = oracle.select(p, q, k, pyr, rows=rows)
    assert np.array_equal(idd, ip)
    np.testing.assert_array_equal(sd, sp)


@pytest.mark.parametrize("scorer,g", [(PISA1, 2), (PISA2, 2), (PISA2, 3)])
def test_pisa_matches_independent_numpy_walk(scorer, g):
    N, K = 2048 + 50, 4
    p, q, k = _prefill(87 + g, N, 2, 1, 16, K, g=g)
    p = replace(p, scorer=scorer)
    pyr = oracle.build_pyramid(p, k)
    rows = list(range(0, N, 41)) + [N - 1]
    idx, _ = oracle.select(p, q, k, pyr, rows=rows)
    kd = k[0, 0].astype(np.float64)
    for t, i in enumerate(rows):
        wi, ws = select_one(q[0, :, i].astype(np.float64), kd, i, 64, K, g, p.s, scorer=scorer)
        if idx[t].tolist() != wi:
            st, _ = oracle.check(p, q, k, pyr, [i], np.array([wi]), np.array([ws], dtype=np.float32),
                                 tau=1e-9, rtol=1e-9)
            assert st[0] == 0, (i, idx[t], wi)


# ------------------------------------------------------- BSA full-scan baseline
# The selector the pages compare against scores every causal block by the dot product with
# its mean-pooled keys ("Block Sparse Attention with Log-Linear Complexity": agihunt.info
# opening and baselines paragraphs; rcap.io picking-step and comparison-point paragraphs).

def test_bsa_score_is_mean_of_raw_key_dots():
    # linearity: the dot with a block's mean is the mean of the dots with its keys (the
    # short last block included), summed over the group's heads
    N, K = 64 * 30 + 21, 8
    p, q, k = _prefill(90, N, 4, 2, 16, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    for row in (N - 1, 2 * N + 700, 4 * N - 1, 3 * N + 64 * 12):
        bh, i = divmod(row, N)
        b, h = divmod(bh, 2)
        sc = oracle.bsa_scores(p, q, pyr, row)
        assert len(sc) == i // 64 + 1
        kd = k[b, h].astype(np.float64)
        qd = q[b, 2 * h:2 * h + 2, i].astype(np.float64)
        for j in range(len(sc)):
            keys = kd[64 * j:min(64 * j + 64, N)]
            expect = p.s * (keys @ qd.T).mean(axis=0).sum()
            assert abs(sc[j] - expect) < 1e-12 * max(1.0, abs(expect))


def test_bsa_score_below_block_lse():
    # Jensen: per head, s<q, mean_j> <= LSE over block j's keys - log C (complete past blocks)
    N, K = 64 * 24, 8
    p, q, k = _prefill(91, N, 2, 1, 16, K)
    pyr = oracle.build_pyramid(p, k)
    i = N - 1
    p1 = oracle.Problem(1, N, 1, 1, 16, 64, K, 2, dtype=F32)
    for r in range(2):
        qr = np.ascontiguousarray(q[:, r:r + 1])
        sc = oracle.bsa_scores(p1, qr, pyr, i)
        for j in range(i // 64):
            lse, _ = oracle.leaf_score(p1, qr, k, i, j)
            assert sc[j] <= lse - math.log(64) + 1e-12


def test_bsa_selection_is_forced_plus_top_scores():
    N, K = 64 * 40 + 5, 7
    p, q, k = _prefill(92, N, 2, 1, 16, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    rows = list(range(0, 2 * N, 23)) + [N - 1, 2 * N - 1]
    idx, sc = oracle.bsa_select(p, q, pyr, rows=rows)
    for t, row in enumerate(rows):
        b = (row % N) // 64
        forced = {f for f in (0, b - 1, b) if f >= 0}
        n = int((idx[t] >= 0).sum())
        assert n == min(K, b + 1)
        sel = idx[t, :n].tolist()
        assert sel == sorted(sel) and forced <= set(sel)
        assert np.all(idx[t, n:] == -1) and np.all(np.isneginf(sc[t, n:]))
        allsc = oracle.bsa_scores(p, q, pyr, row)
        rest = [j for j in range(b + 1) if j not in forced]
        # brute force: rank the non-forced blocks by (score desc, index asc) with python's sort
        want = sorted(sorted(rest, key=lambda j: (-allsc[j], j))[:K - len(forced)])
        assert sorted(set(sel) - forced) == want
        for u, j in enumerate(sel):
            assert (sc[t, u] == math.inf) if j in forced else (sc[t, u] == allsc[j])


def test_bsa_shift_of_all_keys_shifts_every_score():
    # adding one vector c to every key adds sum_h s<q_h, c> to every block score: the
    # selection is unchanged
    N, K = 64 * 33, 6
    p, q, k = _prefill(93, N, 2, 1, 16, K)
    c = np.random.default_rng(5).standard_normal(16).astype(np.float32)
    k2 = (k + c).astype(np.float32)
    pyr, pyr2 = oracle.build_pyramid(p, k), oracle.build_pyramid(p, k2)
    rows = list(range(64 * 5, N, 97)) + [N - 1]
    i1, s1 = oracle.bsa_select(p, q, pyr, rows=rows)
    i2, s2 = oracle.bsa_select(p, q, pyr2, rows=rows)
    assert np.array_equal(i1, i2)
    for t, row in enumerate(rows):
        shift = p.s * float(q[0, :, row].astype(np.float64).sum(axis=0) @ c.astype(np.float64))
        fin = np.isfinite(s1[t])
        np.testing.assert_allclose(s2[t, fin] - s1[t, fin], shift, atol=1e-6)  # k + c rounds in fp32


def test_bsa_ties_go_to_the_lower_block():
    # blocks with identical keys tie exactly; the lower index wins
    N, K, d = 64 * 20, 5, 8
    r = np.random.default_rng(6)
    k = r.standard_normal((1, 1, N, d)).astype(np.float32)
    for j in (3, 7, 11, 15):
        k[0, 0, 64 * j:64 * j + 64] = k[0, 0, 64 * 5:64 * 5 + 64] + 0.0
    k[0, 0, 64 * 5:64 * 5 + 64] += 3.0  # make the tied blocks' common mean large
    for j in (3, 7, 11, 15):
        k[0, 0, 64 * j:64 * j + 64] = k[0, 0, 64 * 5:64 * 5 + 64]
    q = np.ones((1, 1, N, d), dtype=np.float32)
    p = oracle.Problem(1, N, 1, 1, d, 64, K, 2, dtype=F32)
    pyr = oracle.build_pyramid(p, k)
    idx, _ = oracle.bsa_select(p, q, pyr, rows=[N - 1])
    # forced {0, 18, 19}; two slots among the five tied blocks 3, 5, 7, 11, 15
    assert idx[0].tolist() == [0, 3, 5, 18, 19]


def test_bsa_small_K_and_short_prefixes():
    N, K = 64 * 12, 3
    p, q, k = _prefill(94, N, 1, 1, 16, K)
    pyr = oracle.build_pyramid(p, k)
    idx, sc = oracle.bsa_select(p, q, pyr)
    for i in range(N):
        b = i // 64
        want = sorted({0, b - 1, b} - {-1})
        assert idx[i, :len(want)].tolist() == want and np.all(idx[i, len(want):] == -1)
    K = 16  # K >= every causal block: all of them
    p = oracle.Problem(1, N, 1, 1, 16, 64, K, 2, dtype=F32)
    idx, sc = oracle.bsa_select(p, q, pyr)
    for i in range(0, N, 7):
        b = i // 64
        assert idx[i, :b + 1].tolist() == list(range(b + 1)) and np.all(idx[i, b + 1:] == -1)


def test_bsa_gqa_and_decode():
    N, K = 4096 + 11, 8
    p1, q1, k = _prefill(95, N, 1, 1, 16, K)
    pyr = oracle.build_pyramid(p1, k)
    G = 4
    pG = oracle.Problem(1, N, G, 1, 16, 64, K, 2, dtype=F32)
    qG = np.ascontiguousarray(np.repeat(q1, G, axis=1))
    rows = list(range(0, N, 31))
    i1, s1 = oracle.bsa_select(p1, q1, pyr, rows=rows)
    iG, sG = oracle.bsa_select(pG, qG, pyr, rows=rows)
    assert np.array_equal(i1, iG)
    fin = np.isfinite(s1)
    np.testing.assert_allclose(sG[fin], G * s1[fin], rtol=1e-12)
    # decode = the last prefill row
    p, q, k = _prefill(96, N, 4, 2, 16, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    idd, sd = oracle.bsa_select(p, np.ascontiguousarray(q[:, :, N - 1, :]), pyr, decode=True)
    ip, sp = oracle.bsa_select(p, q, pyr, rows=[(b * 2 + h) * N + N - 1 for b in range(2) for h in range(2)])
    assert np.array_equal(idd, ip)
    np.testing.assert_array_equal(sd, sp)


def test_bsa_checker_accepts_oracle_and_rejects_swaps():
    N, K = 64 * 50, 8
    p, q, k = _prefill(97, N, 2, 1, 16, K)
    pyr = oracle.build_pyramid(p, k)
    rows = list(range(64 * 10, N, 53))
    idx, sc = oracle.bsa_select(p, q, pyr, rows=rows)
    assert np.all(oracle.bsa_check(p, q, pyr, rows, idx, sc, tau=0.0, rtol=1e-6) == 0)
    bad = idx.copy()
    for t, row in enumerate(rows):
        b = row // 64
        allsc = oracle.bsa_scores(p, q, pyr, row)
        out = [j for j in range(1, b - 1) if j not in bad[t]]
        worst = min(out, key=lambda j: allsc[j])
        u = next(u for u in range(K) if bad[t, u] not in (0, b - 1, b))
        bad[t, u] = worst
        bad[t] = np.sort(bad[t])
    st = oracle.bsa_check(p, q, pyr, rows, bad, np.where(np.isinf(sc), sc, 0.0), tau=1e-3, rtol=1e3)
    assert np.all(st == 4)


# ------------------------------------------------- block-sparse attention (consumer)
# Each query attends the keys of its selected blocks ("Block Sparse Attention with
# Log-Linear Complexity": agihunt.info opening paragraph; rcap.io first paragraphs).

def _attn_inputs(seed, N, Hq, Hkv, d, K, B=1):
    w = synth.custom(batch=B, seq_len=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, top_k=K, dtype=F32, seed=seed,
                     needles=2)
    q, k, _ = synth.make_inputs(w)
    v = synth.make_values(w)
    return oracle.Problem(B, N, Hq, Hkv, d, 64, K, 2, dtype=F32), q, k, v


def test_attention_over_every_block_is_causal_attention():
    # selecting every causal block reduces to dense causal attention (torch's fp64 routine)
    import torch
    N, d, K = 64 * 6 + 10, 16, 8
    p, q, k, v = _attn_inputs(100, N, 2, 1, d, K)
    idx = np.full((N, K), -1, dtype=np.int32)
    for i in range(N):
        b = i // 64
        idx[i, :b + 1] = np.arange(b + 1)
    out, lse = oracle.attention(p, q, k, v, idx)
    qt = torch.from_numpy(q[0].astype(np.float64))
    kt = torch.from_numpy(k[0].astype(np.float64)).expand(2, N, d)
    vt = torch.from_numpy(v[0].astype(np.float64)).expand(2, N, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=p.s)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref.numpy(), rtol=1e-10, atol=1e-12)
    logits = p.s * torch.einsum("hid,hjd->hij", qt, kt)
    logits = logits.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse.T, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-10)


def test_attention_special_values():
    N, d, K = 64 * 8, 16, 4
    p, q, k, v = _attn_inputs(101, N, 2, 1, d, K)
    idx = np.full((N, K), -1, dtype=np.int32)
    for i in range(N):
        b = i // 64
        idx[i, :3] = sorted({0, max(b - 1, 0), b})[:3] + [-1] * (3 - len({0, max(b - 1, 0), b}))
    # constant values: the output is that constant
    vc = np.ascontiguousarray(np.broadcast_to(np.arange(d, dtype=np.float32), v.shape))
    out, _ = oracle.attention(p, q, k, vc, idx)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(d), out.shape), rtol=0, atol=1e-12)
    # a query whose only visible key is its own: out = that value, lse = its scaled dot
    one = np.full((1, K), -1, dtype=np.int32)
    one[0, 0] = 3
    out, lse = oracle.attention(p, q, k, v, one, rows=[64 * 3])
    np.testing.assert_allclose(out[0], np.broadcast_to(v[0, 0, 64 * 3], (2, d)), rtol=0, atol=1e-12)
    for r in range(2):
        dot = p.s * float(q[0, r, 64 * 3].astype(np.float64) @ k[0, 0, 64 * 3].astype(np.float64))
        assert abs(lse[0, r] - dot) < 1e-12


def test_attention_ignores_order_padding_and_future_blocks():
    N, d, K = 64 * 10, 16, 6
    p, q, k, v = _attn_inputs(102, N, 4, 2, d, K, B=2)
    rows = [64 * 7 + 5, N + 64 * 9 + 63, 3 * N + 100]
    base = np.array([[0, 2, 5, 6, 7, -1], [0, 1, 4, 8, 9, -1], [0, 1, -1, -1, -1, -1]], dtype=np.int32)
    o1, l1 = oracle.attention(p, q, k, v, base, rows=rows)
    shuffled = np.array([[7, -1, 5, 0, 6, 2], [9, 8, -1, 4, 1, 0], [-1, 1, -1, 0, -1, -1]], dtype=np.int32)
    o2, l2 = oracle.attention(p, q, k, v, shuffled, rows=rows)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    future = base.copy()
    future[:, 5] = [8, 10, 3]  # blocks after the query's own are not attended (row 3: i = 100, b = 1)
    future[2, 2] = 2
    o3, l3 = oracle.attention(p, q, k, v, future, rows=rows)
    np.testing.assert_allclose(o3, o1, rtol=0, atol=0)
    np.testing.assert_allclose(l3, l1, rtol=0, atol=0)


def test_attention_lse_and_weights_from_scipy():
    N, d, K = 64 * 5, 16, 4
    p, q, k, v = _attn_inputs(103, N, 2, 1, d, K)
    i = 64 * 4 + 17
    sel = np.array([[0, 2, 3, 4]], dtype=np.int32)
    out, lse = oracle.attention(p, q, k, v, sel, rows=[i])
    keys = [t for j in (0, 2, 3, 4) for t in range(64 * j, min(64 * j + 64, i + 1))]
    for r in range(2):
        x = p.s * (k[0, 0, keys].astype(np.float64) @ q[0, r, i].astype(np.float64))
        z = float(logsumexp(x))
        assert abs(lse[0, r] - z) < 1e-12
        np.testing.assert_allclose(out[0, r], np.exp(x - z) @ v[0, 0, keys].astype(np.float64), rtol=1e-10,
                                   atol=1e-12)


def test_attention_on_the_selection_gqa_and_decode():
    N, d, K = 4096 + 5, 16, 8
    p, q, k, v = _attn_inputs(104, N, 4, 2, d, K, B=2)
    pyr = oracle.build_pyramid(p, k)
    rows = [(bh * N) + N - 1 for bh in range(4)]
    idx, _ = oracle.select(p, q, k, pyr, rows=rows)
    out, lse = oracle.attention(p, q, k, v, idx, rows=rows)
    # each query head on its own (a one-head problem) gives that head's output
    for t, row in enumerate(rows):
        bh, i = divmod(row, N)
        b, h = divmod(bh, 2)
        for r in range(2):
            p1 = oracle.Problem(1, N, 1, 1, d, 64, K, 2, dtype=F32)
            q1 = np.ascontiguousarray(q[b:b + 1, 2 * h + r:2 * h + r + 1])
            k1 = np.ascontiguousarray(k[b:b + 1, h:h + 1])
            v1 = np.ascontiguousarray(v[b:b + 1, h:h + 1])
            o1, l1 = oracle.attention(p1, q1, k1, v1, idx[t:t + 1], rows=[i])
            np.testing.assert_allclose(o1[0, 0], out[t, r], rtol=0, atol=1e-12)
    # decode = the last prefill row
    qd = np.ascontiguousarray(q[:, :, N - 1, :])
    od, ld = oracle.attention(p, qd, k, v, idx, decode=True)
    np.testing.assert_array_equal(od, out)
    np.testing.assert_array_equal(ld, lse)
