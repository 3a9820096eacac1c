"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of PISA's pyramid Top-K block selector.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``block_selection_pyramid_amd``) never does.

The arithmetic lives in ``pisa_oracle.c`` (plain C, double precision, OpenMP over query
groups); this module only compiles it with gcc and marshals numpy arrays through ctypes.
See the header of ``pisa_oracle.c`` for the passages of the pages each step follows and
for the readings taken where the pages are silent.

Parity pins for every function here live in ``tests/test_oracle_*.py``.  The pruned
routing walk (L >= 2 with K below the number of leaf blocks) has no worked example on
the pages; beyond its invariants and the constructed cases in those tests it is
"parity unpinned" (see the design notes).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pisa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
MAXL = 48

F32, BF16 = 0, 1
# routing-level scorers: the LSE over child summaries and its first- / second-order
# Taylor truncations (PISA-1 / PISA-2)
LSE, PISA1, PISA2 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double semantics).

    ``PISA_ORACLE_LIB`` names another build of this source to load instead (the mutation
    tests use it to load copies with planted mistakes)."""
    alt = os.environ.get("PISA_ORACLE_LIB")
    if alt:
        return alt
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("branch", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("dtype", ctypes.c_int32),
        ("scorer", ctypes.c_int32),
    ]


class _Stats(ctypes.Structure):
    _fields_ = [
        ("levels_scored", ctypes.c_int32),
        ("max_candidates", ctypes.c_int32),
        ("dots", ctypes.c_int64),
        ("min_margin", ctypes.c_double),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.orc_levels.argtypes = [i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp]
        lib.orc_levels.restype = ctypes.c_int
        lib.orc_pyramid_nodes.argtypes = [P]
        lib.orc_pyramid_nodes.restype = i64
        lib.orc_lse.argtypes = [vp, i64]
        lib.orc_lse.restype = ctypes.c_double
        lib.orc_build_pyramid.argtypes = [P, vp, vp]
        lib.orc_select_rows.argtypes = [P, vp, vp, vp, ctypes.c_int32, i64, vp, vp, vp, vp]
        lib.orc_node_score.argtypes = [P, vp, vp, ctypes.c_int32, i64, ctypes.c_int32, i64, vp]
        lib.orc_node_score.restype = ctypes.c_double
        lib.orc_leaf_score.argtypes = [P, vp, vp, ctypes.c_int32, i64, i64, vp]
        lib.orc_leaf_score.restype = ctypes.c_double
        lib.orc_check_rows.argtypes = [
            P, vp, vp, vp, ctypes.c_int32, i64, vp, vp, vp,
            ctypes.c_double, ctypes.c_double, ctypes.c_int32, vp, vp,
        ]
        lib.orc_valid_problem.argtypes = [P]
        lib.orc_bsa_select_rows.argtypes = [P, vp, vp, ctypes.c_int32, i64, vp, vp, vp]
        lib.orc_bsa_scores.argtypes = [P, vp, vp, ctypes.c_int32, i64, vp]
        lib.orc_bsa_scores.restype = i64
        lib.orc_bsa_check_rows.argtypes = [P, vp, vp, ctypes.c_int32, i64, vp, vp, vp, ctypes.c_double,
                                           ctypes.c_double, vp]
        lib.orc_attention_rows.argtypes = [P, vp, vp, vp, ctypes.c_int32, i64, vp, vp, vp, vp]
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Problem:
    """Shape of one selection problem (the same fields the HIP library takes)."""

    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int = 64
    top_k: int = 8
    branch: int = 2
    scale: float = 0.0  # <= 0 selects 1/sqrt(head_dim)
    dtype: int = BF16
    scorer: int = LSE  # routing-level score: LSE, PISA1 or PISA2

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def s(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def c(self) -> _Problem:
        return _Problem(self.batch, self.seq_len, self.n_q_heads, self.n_kv_heads, self.head_dim,
                        self.block, self.top_k, self.branch, self.s, self.dtype, self.scorer)


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_input(p: Problem, a: np.ndarray):
    want = np.float32 if p.dtype == F32 else np.uint16
    if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected contiguous {want.__name__} array, got {a.dtype}")


def levels(N: int, C: int, K: int, g: int) -> list[int]:
    """[n_0 = N, n_1, ..., n_L] as the oracle computes them."""
    buf = np.zeros(MAXL + 2, dtype=np.int64)
    L = _load().orc_levels(N, C, K, g, _ptr(buf))
    return [int(x) for x in buf[: L + 1]]


def pyramid_nodes(p: Problem) -> int:
    return int(_load().orc_pyramid_nodes(ctypes.byref(p.c())))


def valid(p: Problem) -> bool:
    return bool(_load().orc_valid_problem(ctypes.byref(p.c())))


def lse(x) -> float:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return float(_load().orc_lse(_ptr(a), a.size))


def build_pyramid(p: Problem, k: np.ndarray) -> np.ndarray:
    """fp64 pyramid [B, Hkv, T, d], levels 1..L leaf-first."""
    _check_input(p, k)
    T = pyramid_nodes(p)
    out = np.zeros((p.batch, p.n_kv_heads, T, p.head_dim), dtype=np.float64)
    _load().orc_build_pyramid(ctypes.byref(p.c()), _ptr(k), _ptr(out))
    return out


def _rows_arg(rows):
    if rows is None:
        return None, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.size


def select(p: Problem, q: np.ndarray, k: np.ndarray, pyr: np.ndarray | None = None,
           rows=None, decode: bool = False, stats: bool = False):
    """Selection for query groups.

    rows: flat group ids ``(b*Hkv + h)*N + i`` (prefill) or ``b*Hkv + h`` (decode; query at
    position N-1); None = all groups.  Returns idx int32 [n, K], score float64 [n, K]
    (and a structured stats array when ``stats``).
    """
    _check_input(p, q)
    _check_input(p, k)
    if pyr is None:
        pyr = build_pyramid(p, k)
    r, n = _rows_arg(rows)
    if r is None:
        n = p.batch * p.n_kv_heads * (1 if decode else p.seq_len)
    idx = np.zeros((n, p.top_k), dtype=np.int32)
    sc = np.zeros((n, p.top_k), dtype=np.float64)
    st = (_Stats * n)() if stats else None
    rc = _load().orc_select_rows(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(pyr), int(decode), n,
                                 _ptr(r), _ptr(idx), _ptr(sc), st)
    if rc != 0:
        raise ValueError("invalid problem for the oracle: %r" % (p,))
    if not stats:
        return idx, sc
    s = np.array([(x.levels_scored, x.max_candidates, x.dots, x.min_margin) for x in st],
                 dtype=[("levels", "i4"), ("max_cand", "i4"), ("dots", "i8"), ("margin", "f8")])
    return idx, sc, s


def node_score(p: Problem, q: np.ndarray, pyr: np.ndarray, row: int, level: int, j: int,
               decode: bool = False):
    """(sum, per-head) score of node j at level >= 2 for the row's query."""
    ph = np.zeros(p.group, dtype=np.float64)
    v = _load().orc_node_score(ctypes.byref(p.c()), _ptr(q), _ptr(pyr), int(decode), row, level, j,
                               _ptr(ph))
    return v, ph


def leaf_score(p: Problem, q: np.ndarray, k: np.ndarray, row: int, j: int, decode: bool = False):
    """(sum, per-head) causal leaf LSE score of block j for the row's query."""
    ph = np.zeros(p.group, dtype=np.float64)
    v = _load().orc_leaf_score(ctypes.byref(p.c()), _ptr(q), _ptr(k), int(decode), row, j, _ptr(ph))
    return v, ph


CHECK_STATUS = {0: "pass", 1: "shape", 2: "forced-missing", 3: "score", 4: "unreachable",
                5: "inconclusive"}


def check(p: Problem, q: np.ndarray, k: np.ndarray, pyr: np.ndarray, rows, idx: np.ndarray,
          score: np.ndarray, tau: float = 1e-3, rtol: float = 1e-3, max_branches: int = 256,
          decode: bool = False):
    """Tie-tolerant verification of another implementation's selection for ``rows``.

    idx int32 [n, K], score float32 [n, K].  Returns (status int32 [n], branches int32 [n]).
    """
    r, n = _rows_arg(rows)
    if r is None:
        n = p.batch * p.n_kv_heads * (1 if decode else p.seq_len)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(n, p.top_k)
    score = np.ascontiguousarray(score, dtype=np.float32).reshape(n, p.top_k)
    status = np.zeros(n, dtype=np.int32)
    br = np.zeros(n, dtype=np.int32)
    rc = _load().orc_check_rows(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(pyr), int(decode), n, _ptr(r),
                                _ptr(idx), _ptr(score), tau, rtol, max_branches, _ptr(status), _ptr(br))
    if rc != 0:
        raise ValueError("invalid problem for the oracle: %r" % (p,))
    return status, br


# ------------------------------------------------------------------ BSA baseline
# The full-scan selector the pages compare against: every causal leaf block scored by the
# dot product of the queries with its mean-pooled keys (pyramid level 1), heads summed,
# forced blocks as in the pyramid selector (reported with score +inf), Top-(K-|F|) of the
# rest by (score descending, index ascending).

def bsa_select(p: Problem, q: np.ndarray, pyr: np.ndarray, rows=None, decode: bool = False):
    """BSA selection for query groups (rows as for ``select``); idx int32 / score float64 [n, K]."""
    _check_input(p, q)
    r, n = _rows_arg(rows)
    if r is None:
        n = p.batch * p.n_kv_heads * (1 if decode else p.seq_len)
    idx = np.zeros((n, p.top_k), dtype=np.int32)
    sc = np.zeros((n, p.top_k), dtype=np.float64)
    rc = _load().orc_bsa_select_rows(ctypes.byref(p.c()), _ptr(q), _ptr(pyr), int(decode), n, _ptr(r), _ptr(idx),
                                     _ptr(sc))
    if rc != 0:
        raise ValueError("invalid problem for the oracle: %r" % (p,))
    return idx, sc


def bsa_scores(p: Problem, q: np.ndarray, pyr: np.ndarray, row: int, decode: bool = False) -> np.ndarray:
    """Scores of blocks 0..b (every causal block, forced ones included) for one row."""
    out = np.zeros(levels(p.seq_len, p.block, p.top_k, p.branch)[1], dtype=np.float64)
    n = _load().orc_bsa_scores(ctypes.byref(p.c()), _ptr(q), _ptr(pyr), int(decode), row, _ptr(out))
    return out[:n]


def bsa_check(p: Problem, q: np.ndarray, pyr: np.ndarray, rows, idx: np.ndarray, score: np.ndarray,
              tau: float = 1e-3, rtol: float = 1e-3, decode: bool = False) -> np.ndarray:
    """Tie-tolerant verification of another BSA selection; status int32 [n] (codes of ``check``)."""
    r, n = _rows_arg(rows)
    if r is None:
        n = p.batch * p.n_kv_heads * (1 if decode else p.seq_len)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(n, p.top_k)
    score = np.ascontiguousarray(score, dtype=np.float32).reshape(n, p.top_k)
    status = np.zeros(n, dtype=np.int32)
    rc = _load().orc_bsa_check_rows(ctypes.byref(p.c()), _ptr(q), _ptr(pyr), int(decode), n, _ptr(r), _ptr(idx),
                                    _ptr(score), tau, rtol, _ptr(status))
    if rc != 0:
        raise ValueError("invalid problem for the oracle: %r" % (p,))
    return status


# ------------------------------------------------------------ block-sparse attention

def attention(p: Problem, q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, rows=None,
              decode: bool = False):
    """Attention of each row's G query heads over the keys of its selected blocks (idx
    [n, K], entries < 0 or past the query's block skipped, keys causal).  Returns
    out float64 [n, G, d] and lse float64 [n, G]."""
    _check_input(p, q)
    _check_input(p, k)
    _check_input(p, v)
    r, n = _rows_arg(rows)
    if r is None:
        n = p.batch * p.n_kv_heads * (1 if decode else p.seq_len)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(n, p.top_k)
    out = np.zeros((n, p.group, p.head_dim), dtype=np.float64)
    lse = np.zeros((n, p.group), dtype=np.float64)
    rc = _load().orc_attention_rows(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(v), int(decode), n, _ptr(r),
                                    _ptr(idx), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("invalid problem for the oracle: %r" % (p,))
    return out, lse
