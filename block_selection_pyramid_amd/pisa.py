"""Python binding of libpisa (argument marshalling only).

Every step of the selection runs in the HIP kernels of ``libpisa.so``; this module checks
tensor placement/dtype/contiguity, allocates outputs and workspace with torch when the
caller does not pass them, and calls the C ABI declared in ``include/pisa.h`` on torch's
current HIP stream.  There is no CPU fallback: if the library is missing or fails to load,
every call raises.

Names follow the C ABI: ``build_pyramid``, ``select_prefill``, ``select_decode``,
``levels``, ``pyramid_bytes``, ``workspace_bytes``, ``supported``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

from . import build as _build

F32, BF16 = 0, 1
PREFILL, DECODE = 0, 1
LSE, PISA1, PISA2 = 0, 1, 2  # enum pisa_scorer
MAX_LEVELS = 32
# PISA_LIB names another build of the same sources to load instead (the CPU tests load the
# host-sanitized build through it); without it, the in-tree libpisa.so
LIB_PATH = os.environ.get("PISA_LIB") or _build.OUT

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error",
           5: "internal error"}


class PisaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class _CProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("branch", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("scorer", ctypes.c_int32),
    ]


@dataclass(frozen=True)
class Problem:
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int = 64
    top_k: int = 8
    branch: int = 2
    scale: float = 0.0
    dtype: int = BF16
    scorer: int = LSE  # routing-level score: LSE, PISA1 or PISA2 (enum pisa_scorer)

    def c(self) -> _CProblem:
        return _CProblem(self.batch, self.seq_len, self.n_q_heads, self.n_kv_heads, self.head_dim, self.block,
                         self.top_k, self.branch, self.scale, self.dtype, self.scorer)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    @property
    def s(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)


_lib = None

EXPORTS = ("pisa_levels", "pisa_pyramid_layout", "pisa_supported", "pisa_pyramid_bytes", "pisa_workspace_bytes", "pisa_build_pyramid",
           "pisa_select_prefill", "pisa_select_prefill_staged", "pisa_prefill_routed_pairs",
           "pisa_prefill_dense_levels", "pisa_select_decode", "pisa_select_prefill_noalloc",
           "pisa_prefill_workspace_min_bytes",
           "pisa_bsa_select_prefill", "pisa_append_keys", "pisa_select_decode_varlen", "pisa_sparse_attention",
           "pisa_attention_workspace_bytes", "pisa_attention_workspace_min_bytes",
           "pisa_status_string", "pisa_version")


def load(path: str | None = None):
    """Loads libpisa.so (building it first only if no build exists)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        if p != _build.OUT:
            raise FileNotFoundError("PISA_LIB names a missing library: %s" % p)
        _build.build(force=True)
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(_CProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.pisa_levels.argtypes = [P, vp, vp, vp]
    lib.pisa_pyramid_layout.argtypes = [P, vp, vp, vp]
    lib.pisa_supported.argtypes = [P, ctypes.c_int]
    lib.pisa_pyramid_bytes.argtypes = [P]
    lib.pisa_pyramid_bytes.restype = sz
    lib.pisa_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.pisa_workspace_bytes.restype = sz
    lib.pisa_prefill_workspace_min_bytes.argtypes = [P]
    lib.pisa_prefill_workspace_min_bytes.restype = sz
    lib.pisa_build_pyramid.argtypes = [P, vp, vp, vp]
    lib.pisa_select_prefill.argtypes = [P, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.pisa_select_prefill_staged.argtypes = [P, vp, vp, vp, vp, sz, vp, vp, vp, ctypes.c_int32, vp]
    lib.pisa_select_prefill_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.pisa_prefill_routed_pairs.argtypes = [P, vp, sz, vp, vp]
    lib.pisa_prefill_dense_levels.argtypes = [P, vp, vp]
    lib.pisa_select_decode.argtypes = [P, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.pisa_bsa_select_prefill.argtypes = [P, vp, vp, vp, vp, vp]
    lib.pisa_append_keys.argtypes = [P, vp, vp, vp, ctypes.c_int32, vp, vp]
    lib.pisa_select_decode_varlen.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.pisa_sparse_attention.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.pisa_attention_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.pisa_attention_workspace_bytes.restype = sz
    lib.pisa_attention_workspace_min_bytes.argtypes = [P, ctypes.c_int32]
    lib.pisa_attention_workspace_min_bytes.restype = sz
    lib.pisa_status_string.argtypes = [ctypes.c_int]
    lib.pisa_status_string.restype = ctypes.c_char_p
    lib.pisa_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise PisaError(rc, what)


def levels(p: Problem):
    """(L, [n_0..n_L], [offset of level 1..L+1])."""
    n = (ctypes.c_int32)()
    nodes = (ctypes.c_int64 * (MAX_LEVELS + 2))()
    offs = (ctypes.c_int64 * (MAX_LEVELS + 2))()
    _check(load().pisa_levels(ctypes.byref(p.c()), ctypes.byref(n), nodes, offs), "pisa_levels")
    L = n.value
    return L, list(nodes[: L + 1]), list(offs[1: L + 2])


def pyramid_layout(p: Problem):
    """(L, [n_1..n_L], [offset of level 1..L, T]) from pisa_pyramid_layout."""
    n = (ctypes.c_int32)()
    nodes = (ctypes.c_int32 * MAX_LEVELS)()
    offs = (ctypes.c_int64 * (MAX_LEVELS + 1))()
    _check(load().pisa_pyramid_layout(ctypes.byref(p.c()), ctypes.byref(n), nodes, offs), "pisa_pyramid_layout")
    L = n.value
    return L, list(nodes[:L]), list(offs[: L + 1])


def supported(p: Problem, mode: int = PREFILL) -> int:
    return load().pisa_supported(ctypes.byref(p.c()), mode)


def pyramid_bytes(p: Problem) -> int:
    return load().pisa_pyramid_bytes(ctypes.byref(p.c()))


def workspace_bytes(p: Problem, mode: int = PREFILL) -> int:
    return load().pisa_workspace_bytes(ctypes.byref(p.c()), mode)


def prefill_workspace_min_bytes(p: Problem) -> int:
    return load().pisa_prefill_workspace_min_bytes(ctypes.byref(p.c()))


def _dev(t: torch.Tensor, name: str, dtype, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def pyramid_shape(p: Problem):
    """Shape of the fp32 pyramid buffer: [2, B, Hkv, Tp, d] with Tp = T rounded up to a
    multiple of 4 (up to three unused nodes per (b, h)); [0] holds the fp32 means, [1] the
    bf16 hi/lo routing copy (its bytes, see include/pisa.h)."""
    L, nodes, offs = levels(p)
    return (2, p.batch, p.n_kv_heads, (offs[-1] + 3) // 4 * 4, p.head_dim)


def pyramid_means(p: Problem, pyramid: torch.Tensor) -> torch.Tensor:
    """The fp32 means [B, Hkv, T, d] inside a pyramid buffer."""
    L, nodes, offs = levels(p)
    return pyramid[0][:, :, : offs[-1]]


def build_pyramid(p: Problem, k: torch.Tensor, pyramid: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    shape = pyramid_shape(p)
    kp = _dev(k, "k", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    if pyramid is None:
        pyramid = torch.empty(shape, dtype=torch.float32, device=k.device)
    pp = _dev(pyramid, "pyramid", torch.float32, shape)
    _check(load().pisa_build_pyramid(ctypes.byref(p.c()), kp, pp, _stream(stream)), "pisa_build_pyramid")
    return pyramid


def workspace(p: Problem, mode: int = PREFILL, device="cuda") -> torch.Tensor:
    n = workspace_bytes(p, mode)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def select_prefill(p: Problem, q: torch.Tensor, k: torch.Tensor, pyramid: torch.Tensor,
                   ws: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                   out_score: torch.Tensor | None = None, stream=None):
    """Returns (idx int32 [B, Hkv, N, K], score fp32 [B, Hkv, N, K])."""
    oshape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.seq_len, p.head_dim))
    kp = _dev(k, "k", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    if ws is None:
        ws = workspace(p, PREFILL, q.device)
    if out_idx is None:
        out_idx = torch.empty(oshape, dtype=torch.int32, device=q.device)
    if out_score is None:
        out_score = torch.empty(oshape, dtype=torch.float32, device=q.device)
    wp = _dev(ws, "workspace", torch.uint8)
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    _check(load().pisa_select_prefill(ctypes.byref(p.c()), qp, kp, pp, wp, ws.numel(), ip, sp, _stream(stream)),
           "pisa_select_prefill")
    return out_idx, out_score


NOALLOC_SCRATCH_BYTES = 64 << 20  # PISA_NOALLOC_SCRATCH_BYTES


def select_prefill_noalloc(p: Problem, q: torch.Tensor, k: torch.Tensor, pyramid: torch.Tensor,
                           out_idx: torch.Tensor, out_score: torch.Tensor, stream=None):
    """pisa_select_prefill_noalloc: the selection on the library's own device scratch (no
    workspace, nothing allocated); the caller passes the outputs."""
    oshape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.seq_len, p.head_dim))
    kp = _dev(k, "k", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    _check(load().pisa_select_prefill_noalloc(ctypes.byref(p.c()), qp, kp, pp, ip, sp, _stream(stream)),
           "pisa_select_prefill_noalloc")
    return out_idx, out_score


def append_keys(p: Problem, k_cache: torch.Tensor, old_lengths: torch.Tensor, new_lengths: torch.Tensor,
                max_new_keys: int, pyramid: torch.Tensor, stream=None):
    """pisa_append_keys: p.seq_len is the cache capacity; lengths are int32 [B] on the device."""
    kp = _dev(k_cache, "k_cache", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    op = _dev(old_lengths, "old_lengths", torch.int32, (p.batch,))
    np_ = _dev(new_lengths, "new_lengths", torch.int32, (p.batch,))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    _check(load().pisa_append_keys(ctypes.byref(p.c()), kp, op, np_, int(max_new_keys), pp, _stream(stream)),
           "pisa_append_keys")
    return pyramid


def select_decode_varlen(p: Problem, q: torch.Tensor, k_cache: torch.Tensor, pyramid: torch.Tensor,
                         lengths: torch.Tensor, out_idx: torch.Tensor | None = None,
                         out_score: torch.Tensor | None = None, stream=None):
    """pisa_select_decode_varlen: the query of sequence b sits at position lengths[b] - 1 of a
    cache of capacity p.seq_len.  Returns (idx int32 [B, Hkv, K], score fp32 [B, Hkv, K])."""
    oshape = (p.batch, p.n_kv_heads, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.head_dim))
    kp = _dev(k_cache, "k_cache", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    lp = _dev(lengths, "lengths", torch.int32, (p.batch,))
    if out_idx is None:
        out_idx = torch.empty(oshape, dtype=torch.int32, device=q.device)
    if out_score is None:
        out_score = torch.empty(oshape, dtype=torch.float32, device=q.device)
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    _check(load().pisa_select_decode_varlen(ctypes.byref(p.c()), qp, kp, pp, lp, ip, sp, _stream(stream)),
           "pisa_select_decode_varlen")
    return out_idx, out_score


def attention_workspace_bytes(p: Problem, decode: bool = False) -> int:
    """Workspace for one pass over the whole sequence (bf16 prefill; 0 otherwise)."""
    return int(load().pisa_attention_workspace_bytes(ctypes.byref(p.c()), DECODE if decode else PREFILL))


def attention_workspace_min_bytes(p: Problem, decode: bool = False) -> int:
    """Smallest workspace pisa_sparse_attention accepts (passes over 2048-query ranges)."""
    return int(load().pisa_attention_workspace_min_bytes(ctypes.byref(p.c()), DECODE if decode else PREFILL))


def sparse_attention(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                     decode: bool = False, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                     want_lse: bool = True, ws: torch.Tensor | None = None, stream=None):
    """pisa_sparse_attention: returns (out [B, Hq, N, d] or [B, Hq, d] in q's dtype, lse fp32
    [B, Hq, N] or [B, Hq], or None when want_lse is False)."""
    qshape = (p.batch, p.n_q_heads, p.head_dim) if decode else (p.batch, p.n_q_heads, p.seq_len, p.head_dim)
    ishape = (p.batch, p.n_kv_heads, p.top_k) if decode else (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
    kshape = (p.batch, p.n_kv_heads, p.seq_len, p.head_dim)
    qp = _dev(q, "q", p.torch_dtype, qshape)
    kp = _dev(k, "k", p.torch_dtype, kshape)
    vp_ = _dev(v, "v", p.torch_dtype, kshape)
    ip = _dev(idx, "idx", torch.int32, ishape)
    if out is None:
        out = torch.empty(qshape, dtype=p.torch_dtype, device=q.device)
    op = _dev(out, "out", p.torch_dtype, qshape)
    lp = None
    if want_lse:
        if lse is None:
            lse = torch.empty(qshape[:-1], dtype=torch.float32, device=q.device)
        lp = _dev(lse, "lse", torch.float32, qshape[:-1])
    nws = attention_workspace_bytes(p, decode)
    if nws and ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=q.device)
    wp = _dev(ws, "workspace", torch.uint8) if nws else None
    wn = ws.numel() if nws else 0
    _check(load().pisa_sparse_attention(ctypes.byref(p.c()), DECODE if decode else PREFILL, qp, kp, vp_, ip, wp, wn,
                                        op, lp, _stream(stream)), "pisa_sparse_attention")
    return out, (lse if want_lse else None)


def bsa_select_prefill(p: Problem, q: torch.Tensor, pyramid: torch.Tensor, out_idx: torch.Tensor | None = None,
                       out_score: torch.Tensor | None = None, stream=None):
    """Full-scan BSA selection (pisa_bsa_select_prefill); returns (idx int32 [B, Hkv, N, K],
    score fp32 [B, Hkv, N, K]), forced blocks with score +inf."""
    oshape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    if out_idx is None:
        out_idx = torch.empty(oshape, dtype=torch.int32, device=q.device)
    if out_score is None:
        out_score = torch.empty(oshape, dtype=torch.float32, device=q.device)
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    _check(load().pisa_bsa_select_prefill(ctypes.byref(p.c()), qp, pp, ip, sp, _stream(stream)),
           "pisa_bsa_select_prefill")
    return out_idx, out_score


def select_prefill_staged(p: Problem, q, k, pyramid, ws, out_idx, out_score, events, stream=None):
    """pisa_select_prefill recording 6 torch.cuda.Event (enable_timing=True) at its stage
    boundaries (upper-level routing | level-2 routing | group | leaf | forced+final)."""
    oshape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.seq_len, p.head_dim))
    kp = _dev(k, "k", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    wp = _dev(ws, "workspace", torch.uint8)
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    if len(events) != 6:
        raise ValueError("need 6 events")
    arr = (ctypes.c_void_p * 6)(*[e.cuda_event for e in events])
    _check(load().pisa_select_prefill_staged(ctypes.byref(p.c()), qp, kp, pp, wp, ws.numel(), ip, sp, arr, 6,
                                             _stream(stream)), "pisa_select_prefill_staged")
    return out_idx, out_score


def dense_levels(p: Problem) -> tuple[int, int]:
    """(top, bottom) of the levels the bf16 prefill routes densely; (0, 0) if none."""
    top, bot = ctypes.c_int32(), ctypes.c_int32()
    _check(load().pisa_prefill_dense_levels(ctypes.byref(p.c()), ctypes.byref(top), ctypes.byref(bot)),
           "pisa_prefill_dense_levels")
    return top.value, bot.value


def routed_pairs(p: Problem, ws: torch.Tensor, stream=None) -> int:
    """Blocking diagnostic: (query group, leaf block) pairs routed to leaf scoring."""
    out = ctypes.c_int64()
    _check(load().pisa_prefill_routed_pairs(ctypes.byref(p.c()), _dev(ws, "workspace", torch.uint8), ws.numel(),
                                            ctypes.byref(out), _stream(stream)), "pisa_prefill_routed_pairs")
    return out.value


def select_decode(p: Problem, q: torch.Tensor, k_cache: torch.Tensor, pyramid: torch.Tensor,
                  ws: torch.Tensor | None = None, out_idx: torch.Tensor | None = None,
                  out_score: torch.Tensor | None = None, stream=None):
    """Returns (idx int32 [B, Hkv, K], score fp32 [B, Hkv, K]) for the query at N-1."""
    oshape = (p.batch, p.n_kv_heads, p.top_k)
    qp = _dev(q, "q", p.torch_dtype, (p.batch, p.n_q_heads, p.head_dim))
    kp = _dev(k_cache, "k_cache", p.torch_dtype, (p.batch, p.n_kv_heads, p.seq_len, p.head_dim))
    pp = _dev(pyramid, "pyramid", torch.float32, pyramid_shape(p))
    nws = workspace_bytes(p, DECODE)
    wp, wn = None, 0
    if ws is not None:
        wp, wn = _dev(ws, "workspace", torch.uint8), ws.numel()
    elif nws:
        ws = workspace(p, DECODE, q.device)
        wp, wn = ws.data_ptr(), ws.numel()
    if out_idx is None:
        out_idx = torch.empty(oshape, dtype=torch.int32, device=q.device)
    if out_score is None:
        out_score = torch.empty(oshape, dtype=torch.float32, device=q.device)
    ip = _dev(out_idx, "out_idx", torch.int32, oshape)
    sp = _dev(out_score, "out_score", torch.float32, oshape)
    _check(load().pisa_select_decode(ctypes.byref(p.c()), qp, kp, pp, wp, wn, ip, sp, _stream(stream)),
           "pisa_select_decode")
    return out_idx, out_score


def version() -> str:
    return load().pisa_version().decode()
