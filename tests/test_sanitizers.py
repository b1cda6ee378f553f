"""The oracle and the library's host code (argument checks, descriptor preparation, the
knapsack, sizes) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Each build is loaded into a fresh Python process that preloads the matching sanitizer runtime
(g++'s for the oracle, clang's for the library, whose host code hipcc compiles), and the CPU
tests that exercise it run there: any invalid access or undefined operation aborts that process.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(env_extra, preload, tests):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", LD_PRELOAD=preload, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


def test_oracle_under_asan_ubsan():
    lib = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(lib):
        pytest.skip("g++ has no ASan runtime")
    env = dict(os.environ, ORACLE_SANITIZE="1")
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT, env=env, check=True)
    run({"ORACLE_SANITIZE": "1"}, lib,
        ["tests/test_oracle_pins.py", "tests/test_alloc.py", "tests/test_littlebit_pins.py"])


def test_library_host_code_under_asan_ubsan():
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no clang ASan runtime or hipcc")
    env = dict(os.environ, QLINEAR_SANITIZE="1")
    subprocess.run([sys.executable, "-c", "from decode_gemv_thinkbit_amd import build as b; b.build()"], cwd=ROOT,
                   env=env, check=True, capture_output=True)
    run({"QLINEAR_SANITIZE": "1"}, rts[0], ["tests/test_abi.py", "tests/test_alloc.py"])
