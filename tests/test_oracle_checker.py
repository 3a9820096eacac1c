"""The tie-tolerant selection checker (oracle.check) accepts exactly what it should.

Parity rule (from the build's target): selected block-index sets bit-exact except where
the oracle's K-th and (K+1)-th scores differ by less than tau = 1e-3; scores within 1e-3
relative.  These tests feed the checker the oracle's own output, legitimate tie swaps, and
planted mistakes.
"""
import math

import numpy as np

import oracle
from block_selection_pyramid_amd import synth

F32, BF16 = oracle.F32, oracle.BF16


def _setup(N=4096, K=8, Hq=4, Hkv=2, d=32, dtype=BF16, seed=5):
    w = synth.custom(seq_len=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, top_k=K, dtype=dtype, seed=seed,
                     needles=8)
    q, k, _ = synth.make_inputs(w)
    p = oracle.Problem(1, N, Hq, Hkv, d, 64, K, 2, dtype=dtype)
    return p, q, k, oracle.build_pyramid(p, k)


def test_accepts_own_output():
    p, q, k, pyr = _setup()
    rows = np.arange(0, p.n_kv_heads * p.seq_len, 11)
    idx, sc = oracle.select(p, q, k, pyr, rows=rows)
    st, br = oracle.check(p, q, k, pyr, rows, idx, sc.astype(np.float32))
    assert np.all(st == 0), np.bincount(st)
    assert br.min() >= 1


def test_rejects_planted_mistakes():
    p, q, k, pyr = _setup()
    N, K = p.seq_len, p.top_k
    rows = [N - 1, N - 500, 3 * 64 + 10]
    idx, sc = oracle.select(p, q, k, pyr, rows=rows)
    sc = sc.astype(np.float32)

    def status(i2, s2, r=0):
        return oracle.check(p, q, k, pyr, [rows[r]], i2[None], s2[None])[0][0]

    i0, s0 = idx[0].copy(), sc[0].copy()
    b = (N - 1) // 64
    # score perturbed beyond 1e-3 relative
    s1 = s0.copy(); s1[1] *= 1.01
    assert status(i0, s1) == 3
    # a small perturbation within tolerance is fine
    s1 = s0.copy(); s1[1] *= 1 + 2e-4
    assert status(i0, s1) == 0
    # unsorted / duplicated / out-of-range
    i1 = i0.copy(); i1[[1, 2]] = i1[[2, 1]]
    assert status(i1, s0) == 1
    i1 = i0.copy(); i1[2] = i1[1]
    assert status(i1, s0) == 1
    # forced block b-1 replaced by some other block: forced missing
    i1 = i0.copy(); pos = list(i1).index(b - 1)
    other = next(j for j in range(1, b) if j not in i1)
    i1[pos] = other
    o = np.argsort(i1); i1 = i1[o]; s1 = s0[o]
    s1[list(i1).index(other)] = oracle.leaf_score(p, q, k, rows[0], other)[0]
    assert status(i1, s1) == 2
    # a routed block swapped for a block with the right score but never reachable /
    # clearly worse: selection rejected
    routed = [j for j in i0 if j not in (0, b - 1, b)]
    bad = next(j for j in range(1, b - 1) if j not in i0)
    i1 = i0.copy(); i1[list(i1).index(routed[0])] = bad
    o = np.argsort(i1); i1 = i1[o]
    s1 = np.array([oracle.leaf_score(p, q, k, rows[0], int(j))[0] for j in i1], dtype=np.float32)
    assert status(i1, s1) == 4
    # wrong padding
    i2, s2 = idx[2].copy(), sc[2].copy()
    assert (i2 == -1).sum() == K - 4
    s2b = s2.copy(); s2b[-1] = 0.0
    assert status(i2, s2b, 2) == 1


def test_accepts_tie_swaps_and_only_them():
    # zero keys: every non-forced full block ties exactly; the oracle keeps the lowest
    # indices, any other tie resolution reachable by the walk must be accepted.
    N, K, G = 4096, 8, 2
    p = oracle.Problem(1, N, G, 1, 8, 64, K, 2, dtype=F32)
    q = np.random.default_rng(1).standard_normal((1, G, N, 8)).astype(np.float32)
    k = np.zeros((1, 1, N, 8), dtype=np.float32)
    pyr = oracle.build_pyramid(p, k)
    i = N - 1
    idx, sc = oracle.select(p, q, k, pyr, rows=[i])
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5, 62, 63]
    full = np.float32(G * math.log(64))
    # a different tie resolution: the walk could have kept level-3 nodes 8..15 instead
    alt = np.array([0, 40, 41, 42, 43, 44, 62, 63], dtype=np.int32)
    st, br = oracle.check(p, q, k, pyr, [i], alt[None], np.full((1, K), full, dtype=np.float32))
    assert st[0] == 0 and br[0] >= 1
    # with tau = 0 exact ties are still ties (kept >= dropped - 0)
    st, _ = oracle.check(p, q, k, pyr, [i], alt[None], np.full((1, K), full, dtype=np.float32), tau=0.0)
    assert st[0] == 0
    # a set no walk can produce: 5 routed blocks spread over different level-2 subtrees is
    # fine, but selecting 6 routed blocks (one forced dropped) is not
    bad = np.array([0, 1, 2, 3, 4, 5, 6, 63], dtype=np.int32)
    st, _ = oracle.check(p, q, k, pyr, [i], bad[None], np.full((1, K), full, dtype=np.float32))
    assert st[0] == 2


def test_decode_rows():
    p, q, k, pyr = _setup(N=4096 + 5, Hq=4, Hkv=2)
    qd = np.ascontiguousarray(q[:, :, -1, :])
    idx, sc = oracle.select(p, qd, k, pyr, decode=True)
    st, _ = oracle.check(p, qd, k, pyr, None, idx, sc.astype(np.float32), decode=True)
    assert np.all(st == 0)
