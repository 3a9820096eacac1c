"""CPU checks of the C ABI: the library loads, exports every function include/pisa.h
declares, and rejects bad arguments on the host before any HIP call (no compute call
here ever passes validation, so nothing touches a GPU)."""
import ctypes
import os
import re

import pytest

import oracle
from block_selection_pyramid_amd import build as pbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pisa.h")


@pytest.fixture(scope="module")
def pisa():
    from block_selection_pyramid_amd import pisa as m
    m.load()
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pisa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_entry_points():
    fns = declared_functions()
    for f in ("pisa_build_pyramid", "pisa_select_prefill", "pisa_select_decode"):
        assert f in fns


def test_library_exports_every_declared_symbol(pisa):
    lib = pisa.load()
    for f in declared_functions():
        assert hasattr(lib, f), f
    assert set(pisa.EXPORTS) == set(declared_functions())
    # exported names are plain C symbols (extern "C")
    out = os.popen("nm -D --defined-only %s" % pisa.LIB_PATH).read()
    for f in declared_functions():
        assert re.search(r"\bT %s$" % f, out, flags=re.M), f


def test_status_strings_and_version(pisa):
    lib = pisa.load()
    assert lib.pisa_status_string(0) == b"ok"
    assert lib.pisa_status_string(3) == b"workspace too small"
    assert re.match(r"^\d+\.\d+\.\d+$", pisa.version())


@pytest.mark.parametrize("N,K", [(1024, 4), (4096, 8), (16384, 32), (65536, 8), (262144, 8), (1000, 3),
                                 (4096 + 37, 5), (1, 8), (64 * 17, 4)])
def test_level_table_matches_oracle(pisa, N, K):
    p = pisa.Problem(1, N, 4, 1, 128, 64, K, 2)
    L, nodes, offs = pisa.levels(p)
    assert nodes == oracle.levels(N, 64, K, 2)
    assert offs[0] == 0 and offs[-1] == sum(nodes[1:])
    assert pisa.pyramid_bytes(p) == 2 * 4 * ((offs[-1] + 3) // 4 * 4) * 128
    L2, nodes2, offs2 = pisa.pyramid_layout(p)
    assert L2 == L and nodes2 == nodes[1:] and offs2 == offs


def test_decode_k32_at_full_decode_shape_is_supported(pisa):
    # 32 sequences x 256K keys, 16/4 heads: B*Hkv*N*2K = 2^31 is past the prefill list limit,
    # which decode, its pyramid build and the append path do not use
    p = pisa.Problem(32, 262144, 16, 4, 128, 64, 32, 2)
    assert pisa.supported(p, pisa.DECODE) == 0
    assert pisa.supported(p, pisa.PREFILL) == 2


def test_sizes(pisa):
    p = pisa.Problem(1, 262144, 16, 4, 128, 64, 8, 2)
    assert pisa.pyramid_bytes(p) == 2 * 4 * 4 * 8176 * 128
    ws = pisa.workspace_bytes(p, pisa.PREFILL)
    slots = 4 * 262144 * 16
    # candidates, leaf scores and list entries per slot; counts, cursors, offsets and
    # chunk offsets per (KV head, leaf block) list; three forced-block scores per query group
    need = slots * 12 + 4 * 262144 * 3 * 4
    # the level-2 launch's fp8 leaf records: 128 e4m3 bytes and one scale byte per leaf
    lo8 = 4 * 4096 * 129
    qcopy = 16 * 262144 * 128 * 2  # the regrouped query copy (bf16, q's size)
    assert ws >= need + lo8 + qcopy and ws < need + lo8 + qcopy + 4 * 4 * 4096 * 4 + 4096
    wmin = pisa.prefill_workspace_min_bytes(p)
    assert wmin >= need + lo8 and wmin < need + lo8 + 4 * 4 * 4096 * 4 + 4096
    # no copy without a dense routing launch (fp32)
    pf = pisa.Problem(1, 262144, 16, 4, 128, 64, 8, 2, dtype=pisa.F32)
    assert pisa.workspace_bytes(pf, pisa.PREFILL) == pisa.prefill_workspace_min_bytes(pf)
    assert pisa.workspace_bytes(p, pisa.DECODE) == 0


@pytest.mark.parametrize("N,K", [(1024, 4), (4096, 8), (16384, 32), (65536, 8), (131072, 8), (131072 + 64, 8),
                                 (262144, 8), (262144 + 1, 8), (300000, 8), (1 << 20, 8)])
def test_dense_level_split(pisa, N, K):
    # bf16: levels L .. bottom are scored densely, where bottom is the highest level >= 2
    # whose child level has at most 1024 nodes (the top level always qualifies: its
    # child level has at most 2gK <= 64 nodes; bottom = 2 when there are at most 1024 leaf
    # blocks); fp32 and L < 3 have no dense launch
    nodes = oracle.levels(N, 64, K, 2)
    L = len(nodes) - 1
    bf = pisa.Problem(1, N, 4, 1, 128, 64, K, 2, dtype=pisa.BF16)
    top, bot = pisa.dense_levels(bf)
    if L < 3:
        assert (top, bot) == (0, 0)
    else:
        want = min(l for l in range(2, L + 1) if nodes[l - 1] <= 1024 or l == L)
        assert (top, bot) == (L, want)
        assert 2 <= bot <= top
        assert (bot == 2) == (nodes[1] <= 1024)
    assert pisa.dense_levels(pisa.Problem(1, N, 4, 1, 128, 64, K, 2, dtype=pisa.F32)) == (0, 0)


def test_dense_level_split_rejects_bad_arguments(pisa):
    lib = pisa.load()
    p = pisa.Problem(1, 4096, 4, 1, 128, 64, 8, 2)
    t = ctypes.c_int32()
    assert lib.pisa_prefill_dense_levels(ctypes.byref(p.c()), None, ctypes.byref(t)) == 1
    bad = pisa.Problem(1, 0, 4, 1, 128, 64, 8, 2)
    assert lib.pisa_prefill_dense_levels(ctypes.byref(bad.c()), ctypes.byref(t), ctypes.byref(t)) == 1


def _call_prefill(pisa, p, ws_bytes=1 << 40, q=0x1000, k=0x1000, pyr=0x1000, ws=0x1000, oi=0x1000, os_=0x1000):
    lib = pisa.load()
    return lib.pisa_select_prefill(ctypes.byref(p.c()), q, k, pyr, ws, ws_bytes, oi, os_, None)


@pytest.mark.parametrize("field,value", [("batch", 0), ("seq_len", 0), ("n_q_heads", 6), ("n_kv_heads", 0),
                                         ("top_k", 2), ("branch", 1), ("head_dim", 0), ("block", 0),
                                         ("dtype", 7), ("scorer", 3), ("scorer", -1)])
def test_invalid_arguments(pisa, field, value):
    base = dict(batch=1, seq_len=4096, n_q_heads=16, n_kv_heads=4, head_dim=128)
    base[field] = value
    p = pisa.Problem(**base)
    assert pisa.supported(p) == 1
    assert pisa.pyramid_bytes(p) == 0 and pisa.workspace_bytes(p) == 0
    assert _call_prefill(pisa, p) == 1
    lib = pisa.load()
    assert lib.pisa_build_pyramid(ctypes.byref(p.c()), 0x1000, 0x1000, None) == 1
    assert lib.pisa_select_decode(ctypes.byref(p.c()), 0x1000, 0x1000, 0x1000, None, 0, 0x1000, 0x1000, None) == 1
    assert lib.pisa_bsa_select_prefill(ctypes.byref(p.c()), 0x1000, 0x1000, 0x1000, 0x1000, None) == 1


def test_append_and_varlen_host_checks(pisa):
    lib = pisa.load()
    p = pisa.Problem(2, 4096, 16, 4, 128)
    P = ctypes.byref(p.c())
    assert lib.pisa_append_keys(P, 0, 0x1000, 0x1000, 1, 0x1000, None) == 1          # null cache
    assert lib.pisa_append_keys(P, 0x1000, 0x1002, 0x1000, 1, 0x1000, None) == 1     # misaligned lengths
    assert lib.pisa_append_keys(P, 0x1000, 0x1000, 0x1000, -1, 0x1000, None) == 1    # negative count
    assert lib.pisa_append_keys(P, 0x1000, 0x1000, 0x1000, 4097, 0x1000, None) == 1  # beyond capacity
    assert lib.pisa_append_keys(P, 0x1000, 0x1000, 0x1000, 0, 0x1000, None) == 0     # nothing to do
    assert lib.pisa_select_decode_varlen(P, 0x1000, 0x1000, 0x1000, 0, 0x1000, 0x1000, None) == 1
    assert lib.pisa_select_decode_varlen(P, 0x1000, 0x1000, 0x1008, 0x1000, 0x1000, 0x1000, None) == 1
    bad = pisa.Problem(2, 4096, 16, 4, 96)
    assert lib.pisa_select_decode_varlen(ctypes.byref(bad.c()), 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                                         None) == 2


def test_attention_host_checks(pisa):
    lib = pisa.load()
    p = pisa.Problem(1, 4096, 16, 4, 128)
    P = ctypes.byref(p.c())
    need = lib.pisa_attention_workspace_bytes(P, pisa.PREFILL)
    least = lib.pisa_attention_workspace_min_bytes(P, pisa.PREFILL)
    assert 0 < least < need and lib.pisa_attention_workspace_bytes(P, pisa.DECODE) == 0
    f32 = pisa.Problem(1, 4096, 16, 4, 128, dtype=pisa.F32)
    assert lib.pisa_attention_workspace_bytes(ctypes.byref(f32.c()), pisa.PREFILL) == 0
    a = (0x1000, 0x1000, 0x1000, 0x1000)
    assert lib.pisa_sparse_attention(P, pisa.PREFILL, *a, None, need, 0x1000, None, None) == 1       # no workspace
    assert lib.pisa_sparse_attention(P, pisa.PREFILL, *a, 0x1000, least - 1, 0x1000, None, None) == 3  # too small
    assert lib.pisa_sparse_attention(P, 7, *a, 0x1000, need, 0x1000, None, None) == 1                 # bad mode
    assert lib.pisa_sparse_attention(P, pisa.PREFILL, 0, *a[1:], 0x1000, need, 0x1000, None, None) == 1


@pytest.mark.parametrize("B,N,Hq,Hkv,d,K", [(1, 262144, 16, 4, 128, 8), (2, 3000 + 17, 8, 2, 64, 6), (1, 5, 8, 2, 64, 4)])
def test_attention_workspace_regions(pisa, B, N, Hq, Hkv, d, K):
    # bf16 prefill, queries in ranges of R (a multiple of 2048): per slot (K per query group)
    # a candidate and a list entry; per (range, KV head, leaf block) list a count, a cursor,
    # an offset and a chunk offset (+1 each for the offsets); per query group of one range
    # K G log2-sum-exp partials and K G bf16 output rows for the slots, G and G for the
    # forced blocks; ten 256-byte aligned regions.  The full size is one range (R = N
    # rounded up to 2048), the minimum R = 2048.
    lib = pisa.load()
    p = pisa.Problem(B, N, Hq, Hkv, d, 64, K, 2)
    G, BH, n1 = Hq // Hkv, B * Hkv, -(-N // 64)
    slots = BH * N * K

    def need(R):
        nr = -(-N // R)
        return slots * 8 + nr * BH * n1 * 4 * 4 + 2 * 4 + BH * R * (K + 1) * G * (4 + 2 * d)

    full = need(-(-N // 2048) * 2048)
    got = lib.pisa_attention_workspace_bytes(ctypes.byref(p.c()), pisa.PREFILL)
    assert full <= got < full + 10 * 256
    got_min = lib.pisa_attention_workspace_min_bytes(ctypes.byref(p.c()), pisa.PREFILL)
    assert need(2048) <= got_min < need(2048) + 10 * 256
    assert got_min <= got
    if N > 2048:
        assert got_min < got
    # decode and fp32 take no workspace
    assert lib.pisa_attention_workspace_min_bytes(ctypes.byref(p.c()), pisa.DECODE) == 0


def test_bsa_host_checks(pisa):
    lib = pisa.load()
    p = pisa.Problem(1, 4096, 16, 4, 128)
    assert lib.pisa_bsa_select_prefill(ctypes.byref(p.c()), 0, 0x1000, 0x1000, 0x1000, None) == 1
    assert lib.pisa_bsa_select_prefill(ctypes.byref(p.c()), 0x1008, 0x1000, 0x1000, 0x1000, None) == 1
    # fp32 inputs and problems outside the kernels' support matrix
    f32 = pisa.Problem(1, 4096, 16, 4, 128, dtype=pisa.F32)
    assert lib.pisa_bsa_select_prefill(ctypes.byref(f32.c()), 0x1000, 0x1000, 0x1000, 0x1000, None) == 2
    big = pisa.Problem(1, 4096, 16, 4, 128, top_k=33)
    assert lib.pisa_bsa_select_prefill(ctypes.byref(big.c()), 0x1000, 0x1000, 0x1000, 0x1000, None) == 2


def test_null_and_misaligned_pointers(pisa):
    p = pisa.Problem(1, 4096, 16, 4, 128)
    assert _call_prefill(pisa, p, q=0) == 1
    assert _call_prefill(pisa, p, oi=0) == 1
    assert _call_prefill(pisa, p, k=0x1004) == 1
    lib = pisa.load()
    assert lib.pisa_build_pyramid(ctypes.byref(p.c()), 0x1002, 0x1000, None) == 1


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(block=32), dict(branch=3), dict(top_k=33),
                                dict(n_q_heads=12, n_kv_heads=4), dict(n_q_heads=64, n_kv_heads=2)])
def test_unsupported_problems(pisa, kw):
    base = dict(batch=1, seq_len=4096, n_q_heads=16, n_kv_heads=4, head_dim=128)
    base.update(kw)
    p = pisa.Problem(**base)
    assert pisa.supported(p) == 2
    assert _call_prefill(pisa, p) == 2


def test_workspace_too_small(pisa):
    # below the minimum (no room even without the regrouped query copy): rejected on the host
    p = pisa.Problem(1, 4096, 16, 4, 128)
    need = pisa.prefill_workspace_min_bytes(p)
    assert 0 < need < pisa.workspace_bytes(p)
    assert _call_prefill(pisa, p, ws_bytes=need - 1) == 3


def test_binding_rejects_host_tensors(pisa):
    import torch
    p = pisa.Problem(1, 128, 4, 1, 64)
    k = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pisa.build_pyramid(p, k, torch.zeros(1, 1, 3, 64))
