#!/usr/bin/env python3
"""Benchmark of libpisa's pyramid Top-K block selector on one MI355X.

Headline (one "step"): pyramid build + prefill selection at 256K tokens, C=64, K=8, g=2,
16 query / 4 KV heads, d=128, bf16 (the pages' selection-latency workload, synthetic
inputs resident in HBM).  Also timed in the same run: the same step at 64K, and one
decode step (32 sequences x 262144-token cache, precomputed pyramid; cold: each step
follows a 1 GiB write that evicts L2 and MALL; warm: back to back) with, beside it, the
serving-loop step on growing caches (append one key per sequence, then the varlen decode
selection), and the 256K step
with the PISA-1 / PISA-2 routing scorers (ablations; extra fields), block-sparse attention
over that step's selection (the consumer; extra field), and the pyramid
selector against the full-scan BSA selector from 4K to 1M tokens (the pages'
selection-kernel comparison at C=64, K=8, extended past 256K).

Prints one JSON line.  Per-stage times come from HIP events recorded by the library on
the stream its kernels run on (pisa_select_prefill_staged) and around pisa_build_pyramid.
The roofline entry is for the stage with the largest average time, against its binding
roof: the larger of its algorithmic bytes at the HBM peak and its algorithmic flops at the
bf16 MFMA peak (Prefill.work); its HBM traffic comes from the committed counter summary
under profiles/ while the kernel's sources still match it (else null).  ``cpu_baseline`` times the fp64 CPU oracle (test
infrastructure) on a bounded sample of the 256K workload and scales it to the whole
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

METRIC = "pyramid selection latency ms @64K/256K prefill (C=64,K=8); decode µs/step"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# exp2 / log2 issue at a quarter of the fp32 add rate (measured with a throughput loop: 0.25
# against 0.82 wave64 instructions per SIMD per ns); the add rate is 32 lanes per SIMD per
# clock, the figure behind the 157.3 TFLOP/s fp32 vector peak: 256 CUs x 4 SIMDs x 8 x 2.4 GHz
TRANS_PEAK_PER_S = 256 * 4 * 8 * 2.4e9


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-64k", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bsa", action="store_true", help="skip the BSA full-scan crossover timings")
    ap.add_argument("--no-attention", action="store_true", help="skip the block-sparse attention timing")
    ap.add_argument("--no-scorers", action="store_true",
                    help="skip the PISA-1 / PISA-2 ablation timings at 256K")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="query groups the oracle selects for the CPU baseline (0: all 1048576)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, 4K, 16K (K = 32) and 128K prefill timings")
    ap.add_argument("--only", choices=["256k", "64k", "decode", "bsa"], default=None,
                    help="time one workload only (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (reference kernel for HBM counters)")
    return ap.parse_args()


def dev(torch, a):
    t = torch.from_numpy(a)
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def visible(n_l, bq, shift):
    return np.minimum(n_l, (bq >> shift) + 1)


def routing_dots_by_level(levels, K, bq):
    """Child dot products one query (one head) scores at each routing level l = L..2
    (returned as {l: array over queries}).

    Candidates at the top level are its visible nodes; below, the visible children of at
    most K kept nodes (2K slots).  Exact except that a kept frontier node may have one
    visible child instead of two (at most one dot per level less)."""
    L = len(levels) - 1
    out = {}
    if L == 1:
        return out
    cand = visible(levels[L], bq, L - 1)
    for l in range(L, 1, -1):
        vis_child = visible(levels[l - 1], bq, l - 2)
        all_vis = cand == visible(levels[l], bq, l - 1)
        d = np.where(all_vis, vis_child, np.minimum(2 * cand, vis_child))
        out[l] = d
        cand = np.where(cand <= K, d, np.minimum(2 * K, vis_child))
    return out


# Counter summary of the prefill kernels (HBM traffic per launch, FETCH_SIZE and WRITE_SIZE
# scaled by a copy of known size); a stage's figure is valid while the sources of its
# kernel hash to the recorded value.
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "prefill_256k_hbm_traffic.md")
TRAFFIC_SOURCES = {
    "route_upper": ["k_route_dense.hip", "final_dev.h", "route_dev.h", "tile_dev.h", "dev_common.h",
                    "pisa_internal.h"],
    "route_l2": ["k_route_sub.hip", "route_dev.h", "dev_common.h", "pisa_internal.h"],
    "leaf": ["k_leaf.hip", "final_dev.h", "dev_common.h", "pisa_internal.h"],
}


def kernel_sources_sha1(stage):
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_selection_pyramid_amd", "csrc")
    for f in TRAFFIC_SOURCES[stage]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(stage):
    """HBM bytes per launch of a stage's kernel from the committed counter summary, or None
    if there is none or the kernel changed since the counters were taken."""
    if stage not in TRAFFIC_SOURCES:
        return None
    try:
        fields = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if "=" in line and line.lstrip().startswith("- "):
                    k, v = line.lstrip()[2:].split("=", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get(stage + ".sources_sha1") != kernel_sources_sha1(stage):
            return None
        return int(fields[stage + ".hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def forced_keys_per_query(N, C):
    i = np.arange(N)
    bq = i // C
    keys = np.minimum(C, i + 1)                       # block 0 (causal if bq == 0)
    keys = keys + np.where(bq >= 2, C, 0)             # previous block b-1 > 0
    keys = keys + np.where(bq >= 1, i - bq * C + 1, 0)  # current block b > 0
    return keys


class Prefill:
    def __init__(self, torch, pisa, synth, name):
        self.torch, self.pisa = torch, pisa
        self.w = w = synth.WORKLOADS[name]
        t = time.time()
        q, k, _ = synth.make_inputs(w)
        log(f"{name}: inputs generated in {time.time() - t:.1f}s")
        self.q, self.k = dev(torch, q), dev(torch, k)
        del q, k
        self.p = p = pisa.Problem(**w.shape())
        self.pyr = torch.empty(pisa.pyramid_shape(p), dtype=torch.float32, device="cuda")
        self.ws = pisa.workspace(p)
        shape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
        self.oi = torch.empty(shape, dtype=torch.int32, device="cuda")
        self.os = torch.empty(shape, dtype=torch.float32, device="cuda")

    def step(self, ev=None):
        pisa = self.pisa
        if ev is None:
            pisa.build_pyramid(self.p, self.k, self.pyr)
            pisa.select_prefill(self.p, self.q, self.k, self.pyr, self.ws, self.oi, self.os)
            return
        ev[0].record()
        pisa.build_pyramid(self.p, self.k, self.pyr)
        pisa.select_prefill_staged(self.p, self.q, self.k, self.pyr, self.ws, self.oi, self.os, ev[1:7])

    def run(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for e in evs:  # torch creates the HIP event on first record; the library records them later
            for x in e:
                x.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(evs[s])
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        names = ["build", "route_upper", "route_l2", "group", "leaf", "final"]
        stage = {n: [] for n in names}
        for e in evs:
            for j, n in enumerate(names):
                stage[n].append(e[j].elapsed_time(e[j + 1]))
        total = [e[0].elapsed_time(e[6]) for e in evs]
        return wall_ms, {n: statistics.mean(v) for n, v in stage.items()}, statistics.median(total)

    def attention(self, steps, warmup):
        """Block-sparse attention over this step's own selection (values i.i.d. N(0, 1)):
        time per call and the rate at which it moves key and value tiles (2 C d bf16 per
        selected (query group, block) pair)."""
        torch, pisa, w, p = self.torch, self.pisa, self.w, self.p
        from block_selection_pyramid_amd import synth
        v = dev(torch, synth.make_values(w))
        self.step()
        out = torch.empty_like(self.q)
        lse = torch.empty(self.q.shape[:-1], dtype=torch.float32, device="cuda")
        res = {}
        # the one-pass workspace, then a 2 GiB one (passes over query ranges)
        for tag, nbytes in (("", pisa.attention_workspace_bytes(p)), ("_2gib_ws", min(2 << 30, pisa.attention_workspace_bytes(p)))):
            aws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            for _ in range(warmup):
                pisa.sparse_attention(p, self.q, self.k, v, self.oi, out=out, lse=lse, ws=aws)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                pisa.sparse_attention(p, self.q, self.k, v, self.oi, out=out, lse=lse, ws=aws)
            b.record()
            b.synchronize()
            res["ms" + tag] = round(a.elapsed_time(b) / steps, 4)
            res["workspace_GB" + tag] = round(nbytes / 1e9, 3)
            del aws
        pairs = int((self.oi >= 0).sum().item())
        tile_bytes = pairs * 2 * p.block * p.head_dim * 2
        res.update({"pairs": pairs, "tile_GBps": round(tile_bytes / (res["ms"] * 1e-3) / 1e9, 1)})
        return res

    def work(self):
        """Algorithmic work of each stage for one step: (bytes, flops).  Bytes are the
        unique HBM bytes the stage must move (each input read once, each output written
        once); flops are the walk's dot products (2d per child and head) and the leaf and
        forced-block key dots, however many the kernels execute."""
        p, w = self.p, self.w
        d, G, C, K = p.head_dim, p.n_q_heads // p.n_kv_heads, p.block, p.top_k
        L, levels, offs = self.pisa.levels(p)
        T = offs[-1]
        BH, N = p.batch * p.n_kv_heads, p.seq_len
        esz = 2 if p.dtype == self.pisa.BF16 else 4
        bq = np.arange(N) // C
        by_level = routing_dots_by_level(levels, K, bq)
        top, bot = self.pisa.dense_levels(p)  # (0, 0): every level by gathers
        dense_l = [l for l in by_level if bot and l >= bot]
        gather_l = [l for l in by_level if l not in dense_l]
        dots = lambda ls: int(sum(by_level[l].sum() for l in ls))
        copy = lambda ls: BH * sum(levels[l - 1] for l in ls) * d * 4  # child levels' routing copy
        pairs = self.pisa.routed_pairs(p, self.ws)
        fflops = BH * int(forced_keys_per_query(N, C).sum()) * G * 2 * d
        q_b, k_b = BH * G * N * d * esz, BH * N * d * esz
        slots = BH * N * 2 * K * 4  # one int32 / fp32 per candidate slot
        forced_in_route = bool(bot)
        step_bytes = q_b + 2 * k_b + 2 * BH * T * d * 4 + BH * N * K * 8
        step_flops = (dots(by_level) * BH * G * 2 * d + pairs * G * C * 2 * d + fflops)
        return {
            "_step": (step_bytes, step_flops),
            "_d": d,
            "build": (BH * N * d * esz + BH * T * d * 8, 0),
            "route_upper": ((q_b + k_b + copy(dense_l) + slots + BH * N * 3 * 4, dots(dense_l) * BH * G * 2 * d
                             + fflops) if forced_in_route else (0, 0)),
            # no gathered level: the stage is the leaf-pair count over the candidate slots
            "route_l2": ((q_b + (slots if forced_in_route else 0) + copy(gather_l) + slots,
                          dots(gather_l) * BH * G * 2 * d) if gather_l else (slots, 0)),
            "group": (BH * N * 2 * K * 4 * 4, 0),
            "leaf": (q_b + k_b + 2 * slots, pairs * G * C * 2 * d),
            "final": (BH * N * ((2 * K + 3) * 4 + K * 8) + (0 if forced_in_route else q_b + k_b),
                      0 if forced_in_route else fflops),
            "_pairs": pairs,
        }


def step_roofline(work, ms_per_step):
    """Roofline of the whole step: T_roof = max(unique HBM bytes / HBM peak, the walk's dot
    flops / bf16 MFMA peak, its exponentials / transcendental rate), each kind of work
    charged to the unit that does it fastest; frac = T_roof / measured step time.  Bytes:
    q and k read once, the pyramid written and read once, the outputs written once (k is
    read by the build and again by the leaf and forced stages: 2 k).  Flops: every routing
    child dot, routed leaf key and forced key (2 d per key and head).  Exponentials: one per
    such dot."""
    nbytes, flops = work["_step"]
    exps = flops / (2 * work["_d"])
    t = {"hbm": nbytes / (HBM_PEAK_GBS * 1e9), "mfma": flops / (MFMA_BF16_PEAK_TFLOPS * 1e12),
         "exp": exps / TRANS_PEAK_PER_S}
    bound = max(t, key=t.get)
    return {"bound": bound, "t_roof_ms": round(t[bound] * 1e3, 4), "ms_per_step": round(ms_per_step, 4),
            "frac": round(t[bound] * 1e3 / ms_per_step, 4), "bytes": int(nbytes), "flops": int(flops),
            "exps": int(exps), "t_hbm_ms": round(t["hbm"] * 1e3, 4), "t_mfma_ms": round(t["mfma"] * 1e3, 4),
            "t_exp_ms": round(t["exp"] * 1e3, 4)}


def roofline(stage_ms, work):
    """Roofline of the stage with the largest time: its binding roof is the larger of its
    algorithmic bytes at the HBM peak and its algorithmic flops at the bf16 MFMA peak (each
    kind of work charged to the unit that does it fastest); frac = that time / measured."""
    dom = max((n for n in stage_ms if n in work), key=lambda n: stage_ms[n])
    nbytes, flops = work[dom]
    t = stage_ms[dom] * 1e-3
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12):
        bound, achieved, peak, unit = "hbm", nbytes / t / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    return dom, {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                 "frac": round(achieved / peak, 4), "traffic": recorded_traffic(dom)}


def time_decode(torch, pisa, synth, steps):
    w = synth.WORKLOADS["decode"]
    t = time.time()
    q, k, _ = synth.make_inputs(w)
    log(f"decode: inputs generated in {time.time() - t:.1f}s")
    qd, kd = dev(torch, q), dev(torch, k)
    del q, k
    p = pisa.Problem(**w.shape())
    pyr = pisa.build_pyramid(p, kd)
    oi = torch.empty((p.batch, p.n_kv_heads, p.top_k), dtype=torch.int32, device="cuda")
    os_ = torch.empty((p.batch, p.n_kv_heads, p.top_k), dtype=torch.float32, device="cuda")
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB > L2 + MALL
    for _ in range(5):
        pisa.select_decode(p, qd, kd, pyr, None, oi, os_)
    torch.cuda.synchronize()
    cold = []
    for _ in range(steps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pisa.select_decode(p, qd, kd, pyr, None, oi, os_)
        b.record()
        b.synchronize()
        cold.append(a.elapsed_time(b) * 1e3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        pisa.select_decode(p, qd, kd, pyr, None, oi, os_)
    b.record()
    b.synchronize()
    warm = a.elapsed_time(b) * 1e3 / steps

    # serving-loop step on growing caches: sequence b holds N - 1 - (997 b mod 4096) keys
    # of the same 262144-key cache; a step appends one key per sequence (pisa_append_keys)
    # and selects for the new query at the new length (pisa_select_decode_varlen)
    lens = [p.seq_len - 1 - (997 * x) % 4096 for x in range(p.batch)]
    old = torch.tensor(lens, dtype=torch.int32, device="cuda")
    new = old + 1
    vpyr = torch.zeros_like(pyr)
    pisa.append_keys(p, kd, torch.zeros_like(old), old, max(lens), vpyr)
    torch.cuda.synchronize()

    def step():
        pisa.append_keys(p, kd, old, new, 1, vpyr)
        pisa.select_decode_varlen(p, qd, kd, vpyr, new, oi, os_)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    vcold = []
    for _ in range(steps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        vcold.append(a.elapsed_time(b) * 1e3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    b.synchronize()
    vwarm = a.elapsed_time(b) * 1e3 / steps

    return statistics.median(cold), warm, statistics.median(vcold), vwarm


CROSSOVER_SIZES = [4096, 16384, 65536, 131072, 262144, 524288, 1048576]


def crossover(torch, pisa, synth, steps, warmup):
    """Pyramid selector vs the full-scan BSA selector at C=64, K=8, 16/4 heads, d=128 (the
    pages' selection-kernel comparison), both including the pyramid build (BSA reads its
    level-1 summaries).  Returns {N: {pisa_ms, bsa_ms, bsa_over_pisa}}."""
    out = {}
    for N in CROSSOVER_SIZES:
        name = {65536: "64k", 131072: "128k", 262144: "256k"}.get(N)
        w = synth.WORKLOADS[name] if name else synth.custom(
            name="crossover-%d" % N, batch=1, seq_len=N, n_q_heads=16, n_kv_heads=4, head_dim=128, top_k=8,
            seed=20 + N // 4096, needles=max(N // 256, 1))
        q, k, _ = synth.make_inputs(w)
        qd, kd = dev(torch, q), dev(torch, k)
        del q, k
        p = pisa.Problem(**w.shape())
        pyr = torch.empty(pisa.pyramid_shape(p), dtype=torch.float32, device="cuda")
        ws = pisa.workspace(p)
        shape = (p.batch, p.n_kv_heads, p.seq_len, p.top_k)
        oi = torch.empty(shape, dtype=torch.int32, device="cuda")
        os_ = torch.empty(shape, dtype=torch.float32, device="cuda")

        def run_pisa():
            pisa.build_pyramid(p, kd, pyr)
            pisa.select_prefill(p, qd, kd, pyr, ws, oi, os_)

        def run_bsa():
            pisa.build_pyramid(p, kd, pyr)
            pisa.bsa_select_prefill(p, qd, pyr, oi, os_)

        res = {}
        n_steps = steps if N <= 262144 else max(2, steps // 4)  # the full scan grows as N^2
        for tag, fn in (("pisa", run_pisa), ("bsa", run_bsa)):
            for _ in range(min(warmup, n_steps)):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(n_steps):
                fn()
            b.record()
            b.synchronize()
            res[tag + "_ms"] = round(a.elapsed_time(b) / n_steps, 4)
        res["bsa_over_pisa"] = round(res["bsa_ms"] / res["pisa_ms"], 3)
        out[str(N)] = res
        log("crossover N=%d: %s" % (N, res))
        del qd, kd, pyr, ws, oi, os_
        torch.cuda.empty_cache()
    return out


def extra_rooflines(extra):
    """Roofline fractions of the rows timed beside the headline (algorithmic work per
    launch in the design notes): the full scan at 256K (MFMA: every causal block's summary
    dot, counted once although hi and lo are both contracted), block-sparse attention at
    256K (MFMA: the selected keys' score and value products; its unique bytes are far
    below the HBM roof), and the 32 x 256K decode step (HBM: the walk's node gathers plus
    the scored key tiles and the query rows)."""
    out = {}
    N, Hkv, G, d, C, K = 262144, 4, 4, 128, 64, 8
    cross = extra.get("crossover_c64_k8", {}).get(str(N))
    if cross:
        blocks = int(((np.arange(N) // C) + 1).sum())
        flops = Hkv * blocks * G * 2 * d
        ach = flops / (cross["bsa_ms"] * 1e-3) / 1e12
        out["bsa_256k"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    att = extra.get("attention_256k")
    if att:
        flops = att["pairs"] * C * G * d * 4  # score and value products, 2 flops each
        ach = flops / (att["ms"] * 1e-3) / 1e12
        out["attention_256k"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    dec = extra.get("decode_us_per_step")
    if dec:
        units, L = 32 * Hkv, 9
        per_unit = (L - 1) * 2 * K * 4 * d + (2 * K + 3) * C * d * 2 + G * d * 2
        ach = units * per_unit / (dec * 1e-6) / 1e9
        out["decode_cold"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(ach / HBM_PEAK_GBS, 4)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, sample_rows):
    """The fp64 C oracle (OpenMP over query groups) on the 256K prefill workload: pyramid
    build plus the selection of every query group (or of a random sample, scaled up)."""
    import oracle
    w = synth.WORKLOADS["256k"]
    q, k, _ = synth.make_inputs(w)
    op = oracle.Problem(**w.shape())
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    total_rows = w.batch * w.n_kv_heads * w.seq_len
    full = sample_rows <= 0 or sample_rows >= total_rows
    t0 = time.perf_counter()
    pyr = oracle.build_pyramid(op, k)
    t1 = time.perf_counter()
    if full:
        oracle.select(op, q, k, pyr)
        n_rows = total_rows
    else:
        rows = np.sort(np.random.default_rng(0).choice(total_rows, sample_rows, replace=False))
        oracle.select(op, q, k, pyr, rows=rows)
        n_rows = sample_rows
    t2 = time.perf_counter()
    ms = ((t1 - t0) + (t2 - t1) * total_rows / n_rows) * 1e3
    what = ("every one of the %d query groups" % total_rows if full else
            "%d random query groups of %d, select time scaled by %d/%d" % (n_rows, total_rows, total_rows, n_rows))
    return {"value": round(ms, 1), "unit": "ms", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "fp64 C oracle, 256K prefill (16/4 heads, d = 128, K = 8): full pyramid build + "
                      "selection of %s; measured %.1fs" % (what, t2 - t0)}


def bruteforce_selection(q, k, K, C, s):
    """Brute-force all-leaf selection for one KV head with G query heads (q [G, N, d],
    k [N, d], fp64): every causal block scored by the group-summed causal LSE over its raw
    keys, the forced blocks {0, b-1, b} kept, then the K - |F| best other blocks (score
    descending, lower index first).  Returns a list of sets per query."""
    G, N, d = q.shape
    logits = s * np.einsum("gid,td->git", q, k)  # [G, N, N]
    out = []
    for i in range(N):
        b = i // C
        sc = np.zeros(b + 1)
        for j in range(b + 1):
            x = logits[:, i, j * C:min(i + 1, (j + 1) * C)]
            m = x.max(axis=1, keepdims=True)
            sc[j] = float(np.sum(m[:, 0] + np.log(np.exp(x - m).sum(axis=1))))
        forced = {f for f in (0, b - 1, b) if 0 <= f <= b}
        rest = sorted((j for j in range(b + 1) if j not in forced), key=lambda j: (-sc[j], j))
        out.append(forced | set(rest[:max(0, K - len(forced))]))
    return out


def tiny_diagnostics(torch, pisa, synth):
    """The tiny workload (1024 tokens, 16 leaf blocks, K = 4, fp32): how much of the
    brute-force all-leaf ranking the pruned walk on the GPU keeps (recall averaged over query
    positions), and how often each planted needle's block is selected by the query it was
    planted for, by the walk and by brute force."""
    w = synth.WORKLOADS["tiny"]
    q, k, needles = synth.make_inputs(w)
    p = pisa.Problem(**w.shape())
    qd, kd = dev(torch, q), dev(torch, k)
    pyr = pisa.build_pyramid(p, kd)
    idx, _ = pisa.select_prefill(p, qd, kd, pyr)
    idx = idx.cpu().numpy()
    s = 1.0 / np.sqrt(w.head_dim)
    G = w.n_q_heads // w.n_kv_heads
    recall, hits, bf_hits = [], 0, 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            bf = bruteforce_selection(q[b, h * G:(h + 1) * G].astype(np.float64), k[b, h].astype(np.float64),
                                      w.top_k, w.block, s)
            for i in range(w.seq_len):
                got = {int(x) for x in idx[b, h, i] if x >= 0}
                recall.append(len(got & bf[i]) / len(bf[i]))
            for nb, nh, npos, _nq, nj in needles:
                if nb == b and nh == h:
                    hits += int(npos // w.block in set(idx[b, h, nj].tolist()))
                    bf_hits += int(npos // w.block in bf[nj])
    n = max(len(needles), 1)
    return {"recall_vs_bruteforce": round(float(np.mean(recall)), 4), "needles": int(len(needles)),
            "needle_hit_rate": round(hits / n, 4), "needle_hit_rate_bruteforce": round(bf_hits / n, 4)}


def time_config(torch, pisa, synth, name, steps, warmup):
    """Prefill (pyramid build + selection) of one more workload, wall ms per step."""
    b = Prefill(torch, pisa, synth, name)
    wall, stages, _ = b.run(steps, warmup)
    del b
    torch.cuda.empty_cache()
    return round(wall, 4), {k: round(v, 4) for k, v in stages.items()}


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py: this build runs on one GPU only (the selector shards by (batch, KV head) "
              "with no exchange; multi-GPU runs are not part of it); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from block_selection_pyramid_amd import pisa, synth
    pisa.load()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    out = {"metric": METRIC}
    extra = {}
    if a.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    head = None
    if a.only in (None, "256k"):
        b = Prefill(torch, pisa, synth, "256k")
        wall_ms, stage_ms, ev_ms = b.run(a.steps, a.warmup)
        work = b.work()
        dom, roof = roofline(stage_ms, work)
        head = (b.w, wall_ms, stage_ms, ev_ms, dom, roof, work)
        log("256k: wall %.3f ms/step, events %.3f ms; stages %s" % (
            wall_ms, ev_ms, {k: round(v, 3) for k, v in stage_ms.items()}))
        if not a.no_scorers:
            # the PISA-1 / PISA-2 routing scorers on the same inputs (ablations, not the headline)
            from dataclasses import replace
            lse_p = b.p
            for name, scorer in (("pisa1", pisa.PISA1), ("pisa2", pisa.PISA2)):
                b.p = replace(lse_p, scorer=scorer)
                ws, sms, _ = b.run(a.steps, a.warmup)
                extra["prefill_256k_%s_ms" % name] = round(ws, 4)
                extra["prefill_256k_%s_stages_ms" % name] = {k: round(v, 4) for k, v in sms.items()}
                log("256k %s: wall %.3f ms/step; stages %s" % (name, ws, extra["prefill_256k_%s_stages_ms" % name]))
            b.p = lse_p
        if not a.no_attention:
            extra["attention_256k"] = b.attention(a.steps, a.warmup)
            log("256k attention: %s" % extra["attention_256k"])
        del b
        torch.cuda.empty_cache()
    if a.only in (None, "64k") and not a.no_64k:
        b = Prefill(torch, pisa, synth, "64k")
        wall64, stage64, ev64 = b.run(a.steps, a.warmup)
        extra["prefill_64k_ms"] = round(wall64, 4)
        extra["prefill_64k_stages_ms"] = {k: round(v, 4) for k, v in stage64.items()}
        log("64k: wall %.3f ms/step; stages %s" % (wall64, extra["prefill_64k_stages_ms"]))
        del b
        torch.cuda.empty_cache()
    if a.only is None and not a.no_configs:
        # the other prefill workloads: tiny fp32 (K = 4), 4K (K = 8), 16K (K = 32), 128K (K = 8)
        for name in ("tiny", "4k", "16k", "128k"):
            ms, st = time_config(torch, pisa, synth, name, max(a.steps, 20), a.warmup)
            extra["prefill_%s_ms" % name] = ms
            extra["prefill_%s_stages_ms" % name] = st
            log("%s: wall %.3f ms/step; stages %s" % (name, ms, st))
        extra["tiny_diagnostics"] = tiny_diagnostics(torch, pisa, synth)
        log("tiny diagnostics: %s" % extra["tiny_diagnostics"])
    if a.only in (None, "decode") and not a.no_decode:
        cold, warm, vcold, vwarm = time_decode(torch, pisa, synth, a.decode_steps)
        extra["decode_us_per_step"] = round(cold, 2)
        extra["decode_us_per_step_warm"] = round(warm, 2)
        extra["decode_append_varlen_us_per_step"] = round(vcold, 2)
        extra["decode_append_varlen_us_per_step_warm"] = round(vwarm, 2)
        log("decode: cold %.2f us, warm %.2f us; append + varlen decode: cold %.2f us, warm %.2f us" % (
            cold, warm, vcold, vwarm))
        torch.cuda.empty_cache()
    if a.only in (None, "bsa") and not a.no_bsa:
        extra["crossover_c64_k8"] = crossover(torch, pisa, synth, a.steps, a.warmup)
    extra["rooflines"] = extra_rooflines(extra)
    if head is None:
        print(json.dumps(extra))
        return
    w, wall_ms, stage_ms, ev_ms, dom, roof, work = head
    out.update({
        "value": round(wall_ms, 4), "unit": "ms", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall_ms, 4), "higher_is_better": False, "scaling": "strong", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill-256k (pyramid build + selection)", "batch": w.batch, "seq_len": w.seq_len,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block": w.block, "top_k": w.top_k, "branch": w.branch, "parallelism": "single-gpu"},
        "roofline": roof,
        "roofline_kernel": dom,
        "roofline_step": step_roofline(work, wall_ms),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "event_ms_per_step": round(ev_ms, 4),
        "routed_pairs": work["_pairs"],
    })
    out.update(extra)
    if not a.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(synth, a.cpu_sample_rows)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
