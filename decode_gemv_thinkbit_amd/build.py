"""Build libqlinear.so (HIP, gfx950) in-tree: decode_gemv_thinkbit_amd/_build/libqlinear.so."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# QLINEAR_SANITIZE=1: host code built with AddressSanitizer and UndefinedBehaviorSanitizer into
# _build_san/ (device code unchanged); load it in a process that preloads clang's ASan runtime
SANITIZE = os.environ.get("QLINEAR_SANITIZE") == "1"
OUT_DIR = os.path.join(HERE, "_build_san" if SANITIZE else "_build")
LIB = os.path.join(OUT_DIR, "libqlinear.so")
SOURCES = ["ql_api.hip", "ql_pack.hip", "ql_gemv.hip", "ql_gemm.hip", "ql_c4.hip", "ql_alloc.hip", "ql_littlebit.hip", "ql_probe.hip", "ql_noalloc.hip", "ql_check.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep single-lane atomics as written: the wave-aggregating rewrite waits on the
    # grouped GEMV's ticket fetch at once instead of when the ticket is used
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
if SANITIZE:
    FLAGS += ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan", "-g"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if SANITIZE:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
