"""Seeded synthetic inputs shaped like the pages' selection workloads.

The paper's timing runs (the selection kernels alone at C=64 and K=8, 4K-256K tokens)
name no dataset, so every workload here is synthetic: q and k are i.i.d. N(0, 1) from a
counter-based generator (SplitMix64 hash of (seed, tensor id, flat index), then
Box-Muller; see ``csrc/synth.c``), rounded to bf16 with round-to-nearest-even for the
bf16 workloads, plus planted "needle" keys equal to 3x a later query row of a head in
the key head's GQA group.

This module holds no selector arithmetic; both the CPU oracle (in the tests) and the
HIP library read the arrays it returns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

F32, BF16 = 0, 1
TENSOR_Q, TENSOR_K, TENSOR_NEEDLE, TENSOR_BLOCK, TENSOR_V = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    top_k: int
    branch: int
    dtype: int
    seed: int
    needles: int  # per batch row
    decode: bool = False

    def shape(self) -> dict:
        return dict(batch=self.batch, seq_len=self.seq_len, n_q_heads=self.n_q_heads,
                    n_kv_heads=self.n_kv_heads, head_dim=self.head_dim, block=self.block,
                    top_k=self.top_k, branch=self.branch, dtype=self.dtype)


def _wl(name, B, N, Hq, Hkv, d, K, dtype, seed, needles, decode=False):
    return Workload(name, B, N, Hq, Hkv, d, 64, K, 2, dtype, seed, needles, decode)


# The pages' selection workloads: C = 64, g = 2, K = 8 (pretraining) / 32 (16K
# continued pretraining), 4K to 256K tokens; head counts and head dim 128 with GQA
# group 4 as fixed by the workload definitions.  Seeds 1..7 in this order.
WORKLOADS = {
    "tiny": _wl("tiny", 1, 1024, 1, 1, 64, 4, F32, 1, 4),
    "4k": _wl("4k", 1, 4096, 16, 4, 128, 8, BF16, 2, 32),
    "16k": _wl("16k", 1, 16384, 16, 4, 128, 32, BF16, 3, 128),
    "64k": _wl("64k", 1, 65536, 16, 4, 128, 8, BF16, 4, 256),
    "128k": _wl("128k", 1, 131072, 16, 4, 128, 8, BF16, 5, 512),
    "256k": _wl("256k", 1, 262144, 16, 4, 128, 8, BF16, 6, 1024),
    "decode": _wl("decode", 32, 262144, 16, 4, 128, 8, BF16, 7, 256, decode=True),
}


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_round_bf16.argtypes = [vp, i64, vp]
        lib.synth_needles.argtypes = [u64, u64, i32, i32, i32, i64, i32, i32, vp]
        lib.synth_needles.restype = i64
        lib.synth_apply_needles.argtypes = [u64, u64, i32, i32, i32, i64, i32, i32, vp, i64, i32, vp]
        _lib = lib
    return _lib


def _vp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed: int, tensor: int, shape, dtype: int, offset: int = 0) -> np.ndarray:
    """i.i.d. N(0,1) array; float32, or bf16 bit patterns as uint16."""
    n = int(np.prod(shape))
    if dtype == F32:
        out = np.empty(shape, dtype=np.float32)
        _load().synth_normal_f32(seed, tensor, offset, n, _vp(out))
    else:
        out = np.empty(shape, dtype=np.uint16)
        _load().synth_normal_bf16(seed, tensor, offset, n, _vp(out))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); returns the uint16 bit patterns."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_round_bf16(_vp(a), a.size, _vp(out))
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def needle_rows(w: Workload, count: int | None = None) -> np.ndarray:
    """[n, 5] int64 rows (b, kv head, key position p, q head, query position j)."""
    count = w.needles if count is None else count
    buf = np.zeros((max(w.batch * count, 1), 5), dtype=np.int64)
    n = _load().synth_needles(w.seed, TENSOR_NEEDLE, w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len,
                              count, int(w.decode), _vp(buf))
    return buf[:n]


def make_inputs(w: Workload, needles: int | None = None):
    """(q, k, needle_rows) for a workload.

    prefill: q [B, Hq, N, d], k [B, Hkv, N, d]; decode: q [B, Hq, d] (the new token's
    query at position N-1), k [B, Hkv, N, d] (the cache, current token included).
    """
    if w.decode:
        q = normal(w.seed, TENSOR_Q, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    else:
        q = normal(w.seed, TENSOR_Q, (w.batch, w.n_q_heads, w.seq_len, w.head_dim), w.dtype)
    k = normal(w.seed, TENSOR_K, (w.batch, w.n_kv_heads, w.seq_len, w.head_dim), w.dtype)
    rows = needle_rows(w, needles)
    if len(rows):
        _load().synth_apply_needles(w.seed, TENSOR_Q, w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len,
                                    w.head_dim, int(w.decode), _vp(rows), len(rows), w.dtype, _vp(k))
    return q, k, rows


def custom(name: str = "custom", batch=1, seq_len=1024, n_q_heads=4, n_kv_heads=1, head_dim=128,
           block=64, top_k=8, branch=2, dtype=BF16, seed=11, needles=4, decode=False) -> Workload:
    return Workload(name, batch, seq_len, n_q_heads, n_kv_heads, head_dim, block, top_k, branch, dtype,
                    seed, needles, decode)


def add_block_offsets(w: Workload, k: np.ndarray, sigma: float) -> np.ndarray:
    """Keys with a shared offset per leaf block: key t of block b (C = w.block keys) gets
    sigma * v_b added, v_b i.i.d. N(0, 1) per (batch, KV head, block) and dimension, then
    bf16 workloads are rounded again.  The pyramid's means then keep a norm of about
    sigma * sqrt(d) at every level, so sibling nodes' scores lie far apart: the inputs on
    which truncated routing scores visibly depart from the LSE."""
    B, H, N, d = k.shape
    nb = (N + w.block - 1) // w.block
    off = normal(w.seed, TENSOR_BLOCK, (B, H, nb, d), F32) * np.float32(sigma)
    kf = bf16_bits_to_f32(k) if w.dtype == BF16 else k
    kf = kf + np.repeat(off, w.block, axis=2)[:, :, :N, :]
    return to_bf16_bits(kf) if w.dtype == BF16 else np.ascontiguousarray(kf, dtype=np.float32)


def make_values(w: Workload) -> np.ndarray:
    """v [B, Hkv, N, d] (the values block-sparse attention reads), i.i.d. N(0, 1) like k."""
    return normal(w.seed, TENSOR_V, (w.batch, w.n_kv_heads, w.seq_len, w.head_dim), w.dtype)


def random_selection(w: Workload, seed: int, pad: int = 0) -> np.ndarray:
    """A valid selection of the kind the selectors return, drawn at random: int32
    [B, Hkv, N, K] (decode: [B, Hkv, K], the query at N - 1) holding, per row, the existing
    blocks of {0, b - 1, b} and min(K - |F|, b - 2) - pad distinct blocks of 1 .. b - 2,
    ascending, then -1.  Feeds the attention tests without running a selector."""
    rng = np.random.default_rng(seed)
    K, C = w.top_k, w.block
    nq = 1 if w.decode else w.seq_len
    pos = np.full(nq, w.seq_len - 1) if w.decode else np.arange(w.seq_len)
    b = np.tile(pos // C, w.batch * w.n_kv_heads).astype(np.int64)  # leaf block of each row
    nf = np.where(b == 0, 1, np.where(b == 1, 2, 3))
    m = np.clip(np.minimum(K - nf, b - 2) - pad, 0, None)
    R, big = len(b), np.int64(1) << 40
    # m distinct blocks of 1 .. b - 2 without rejection: sorted draws y_0 <= .. <= y_{m-1}
    # from 0 .. b - 2 - m, then x_u = 1 + y_u + u (strictly increasing, at most b - 2)
    room = np.maximum(b - 2 - m + 1, 1)[:, None]
    y = (rng.random((R, K)) * room).astype(np.int64)
    y = np.where(np.arange(K)[None, :] < m[:, None], y, big)
    y.sort(axis=1)
    picks = np.where(y < big, 1 + y + np.arange(K)[None, :], big)
    forced = np.stack([np.zeros(R, np.int64), np.where(b >= 2, b - 1, big), np.where(b >= 1, b, big)], axis=1)
    allv = np.concatenate([forced, picks], axis=1)
    allv.sort(axis=1)
    allv = allv[:, :K]
    out = np.where(allv < big, allv, -1).astype(np.int32)
    shape = (w.batch, w.n_kv_heads, K) if w.decode else (w.batch, w.n_kv_heads, nq, K)
    return out.reshape(shape)
