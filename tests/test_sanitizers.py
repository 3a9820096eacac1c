"""The oracle and libpisa's host code under AddressSanitizer + UndefinedBehaviorSanitizer.

Two CPU-only legs, each in a child process with the sanitizer runtime preloaded:

* the oracle (plain C, gcc) rebuilt with ``-fsanitize=address,undefined`` and loaded through
  ``PISA_ORACLE_LIB`` while the pin and checker suites run;
* libpisa rebuilt with the same sanitizers on its host code only
  (``build(sanitize=True)``, clang's runtime) and loaded through ``PISA_LIB`` while the ABI
  suite runs, so every validation path the ABI tests reach runs instrumented.

UBSan is set to abort on the first report, so any report fails the child.  A control case
per runtime plants a heap overflow in a scratch C file and checks that the same set-up
reports it: a run that passes is then a run the sanitizer actually watched.
"""
import os
import subprocess
import sys
import tempfile

import pytest

from block_selection_pyramid_amd import build as pbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "pisa_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
OVERFLOW_C = "#include <stdlib.h>\nint poke(int n) { int* a = malloc(n * sizeof(int)); a[n] = 1; int r = a[0]; free(a); return r; }\n"


def gcc_asan_runtime():
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def rocm_clang():
    """The clang that hipcc drives (ROCm's llvm/bin next to hipcc's bin/)."""
    c = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(pbuild.hipcc()))), "llvm", "bin", "clang")
    return c if os.path.exists(c) else "/opt/rocm/llvm/bin/clang"


def clang_asan_runtime():
    return subprocess.check_output([rocm_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()


def san_env(runtime, **extra):
    env = dict(os.environ)
    # the runtime must come first; anything already preloaded stays after it
    env["LD_PRELOAD"] = ":".join(x for x in (runtime, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def run_child(args, env, timeout=600):
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def overflow_probe(compiler, runtime, tmp):
    src, lib = os.path.join(tmp, "overflow.c"), os.path.join(tmp, "liboverflow.so")
    with open(src, "w") as f:
        f.write(OVERFLOW_C)
    subprocess.check_call([compiler, "-shared", "-fPIC", *SAN, src, "-o", lib])
    return run_child(["-c", "import ctypes; ctypes.CDLL(%r).poke(4)" % lib], san_env(runtime), timeout=120)


@pytest.fixture(scope="module")
def oracle_san():
    tmp = tempfile.mkdtemp(prefix="oracle_san_")
    lib = os.path.join(tmp, "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-Wall", "-shared", "-fPIC", *SAN, ORACLE_SRC,
                           "-o", lib, "-lm"])
    return tmp, lib


def test_gcc_runtime_reports_a_planted_overflow(oracle_san):
    rc, out = overflow_probe("gcc", gcc_asan_runtime(), oracle_san[0])
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]


def test_oracle_pins_and_checker_under_asan_ubsan(oracle_san):
    rc, out = run_child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                         "tests/test_oracle_pins.py", "tests/test_oracle_checker.py"],
                        san_env(gcc_asan_runtime(), PISA_ORACLE_LIB=oracle_san[1]))
    assert rc == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


@pytest.fixture(scope="module")
def pisa_san():
    return pbuild.build(force=False, sanitize=True)


def test_clang_runtime_reports_a_planted_overflow(pisa_san):
    rc, out = overflow_probe(rocm_clang(), clang_asan_runtime(), tempfile.mkdtemp(prefix="clang_san_"))
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]


def test_abi_suite_on_the_host_sanitized_library(pisa_san):
    rc, out = run_child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"],
                        san_env(clang_asan_runtime(), PISA_LIB=pisa_san))
    assert rc == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
