"""Builds libpisa.so (HIP, gfx950) in-tree with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel), then
linked into ``block_selection_pyramid_amd/libpisa.so``.  Packed-fp32 instructions are
disabled for the device code (``-packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.  Matrix-core results are kept in ordinary
VGPRs (``-amdgpu-mfma-vgpr-form``) so that the epilogues read them without accvgpr
moves.

Every compile also asks for the compiler's per-kernel resource report; the build writes it
to ``_build/kernel_resources.txt`` (VGPRs, scratch bytes per lane, waves per SIMD) and
fails when a kernel instantiation on the 16/4-head, d = 128 bf16 path spills to scratch
(``HEADLINE``): a spill there costs HBM traffic on every launch.

``build(sanitize=True)`` (``--sanitize``) makes a second library,
``_build/san/libpisa_san.so``, whose host code (argument validation, workspace carving,
launch set-up) is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; the
device code is built as usual, without sanitizers.  It needs the ASan runtime preloaded and
is meant for the CPU tests, which load it through ``PISA_LIB``.

Usage: ``python -m block_selection_pyramid_amd.build [--force] [--sanitize] [-j N]``.
"""
from __future__ import annotations

import argparse
import glob
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpisa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("PISA_OFFLOAD_ARCH", "gfx950")

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", CSRC, "-I", INCLUDE,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# host-side sanitizers only: each flag goes to the host compile through -Xarch_host
SAN_FLAGS = [f for x in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                         "-fno-omit-frame-pointer", "-g") for f in ("-Xarch_host", x)]
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_OUT = os.path.join(SAN_DIR, "libpisa_san.so")

RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")

# Kernel instantiations of the d = 128, G = 4 bf16 path (prefill selection and decode) that
# must not spill: demangled-name prefixes.
HEADLINE = (
    "pisa::(anonymous namespace)::route_dense_kernel<128, 4, 8, false>",
    "pisa::(anonymous namespace)::route_sub_kernel<128,",
    "pisa::(anonymous namespace)::lo8_kernel",
    "pisa::(anonymous namespace)::route_mfma_kernel<128, 4,",
    "pisa::(anonymous namespace)::leaf_pair_kernel<128, 4>",
    "pisa::(anonymous namespace)::final_kernel",
    "pisa::(anonymous namespace)::scatter_pairs_hist_kernel",
    "pisa::(anonymous namespace)::pyr_sub_kernel<unsigned short, 128",
    "pisa::(anonymous namespace)::decode_kernel<unsigned short, 128, 4",
)


def _demangle(names: list[str]) -> list[str]:
    exe = shutil.which("c++filt") or shutil.which("llvm-cxxfilt") or "/opt/rocm/llvm/bin/llvm-cxxfilt"
    try:
        r = subprocess.run([exe], input="\n".join(names), capture_output=True, text=True, check=True)
        out = r.stdout.splitlines()
        return out if len(out) == len(names) else names
    except (OSError, subprocess.CalledProcessError):
        return names


def _resources(stderr: str) -> list[tuple[str, int, int, int]]:
    """(kernel, VGPRs, scratch bytes per lane, waves per SIMD) from the compiler remarks."""
    rows, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = [m.group(1), -1, -1, -1]
            rows.append(cur)
            continue
        if cur is None:
            continue
        for i, key in ((1, r"\bVGPRs: (\d+)"), (2, r"ScratchSize \[bytes/lane\]: (\d+)"),
                       (3, r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(key, line)
            if m:
                cur[i] = int(m.group(1))
    names = _demangle([r[0] for r in rows])
    return [(n, r[1], r[2], r[3]) for n, r in zip(names, rows)]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libpisa needs ROCm's hipcc to build")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _deps() -> list[str]:
    return sources() + glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))


def up_to_date(out: str = OUT) -> bool:
    if not os.path.exists(out):
        return False
    t = os.path.getmtime(out)
    return all(os.path.getmtime(p) <= t for p in _deps())


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    extra = SAN_FLAGS if sanitize else []
    cmd = [hipcc(), *CXXFLAGS, *extra, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj, _resources(r.stderr)


def build(force: bool = True, jobs: int | None = None, verbose: bool = False, sanitize: bool = False) -> str:
    """Compiles every HIP source for gfx950 and links libpisa.so (with ``sanitize``, the
    host-sanitized ``_build/san/libpisa_san.so``).  Returns its path."""
    out = SAN_OUT if sanitize else OUT
    if not force and up_to_date(out):
        return out
    os.makedirs(SAN_DIR if sanitize else BUILD_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(lambda s: _compile(s, sanitize), sources()))
    objs = [o for o, _ in done]
    if sanitize:
        return _link(objs, out, SAN_FLAGS, verbose)
    res = sorted(r for _, rs in done for r in rs)
    with open(RESOURCES, "w") as f:
        for name, vgpr, scratch, occ in res:
            f.write("%4d VGPRs %5d B scratch %2d waves/SIMD  %s\n" % (vgpr, scratch, occ, name))
    spills = [r for r in res if r[2] > 0 and r[0].removeprefix("void ").startswith(HEADLINE)]
    if spills:
        raise RuntimeError("headline kernels spill to scratch (see %s):\n%s" % (
            RESOURCES, "\n".join("%d B/lane  %s" % (r[2], r[0]) for r in spills)))
    return _link(objs, OUT, [], verbose)


def _link(objs: list[str], out: str, extra: list[str], verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="build the host-sanitized library instead")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args(argv)
    out = SAN_OUT if a.sanitize else OUT
    build(force=a.force or not up_to_date(out), jobs=a.j, verbose=True, sanitize=a.sanitize)


if __name__ == "__main__":
    sys.exit(main())
