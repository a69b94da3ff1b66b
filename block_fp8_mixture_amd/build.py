"""Builds libmoefp8.so (the HIP kernels and the C ABI) in place, for gfx950.

Usage: python -m block_fp8_mixture_amd.build   (or build() from Python).
Each translation unit is compiled in parallel, then linked into one shared
library next to this file. Compiled without fast-math (IEEE division and
denormals, which the quantizers rely on), with floating-point contraction
off (the kernels write their FMAs explicitly), and with packed fp32
arithmetic disabled.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoefp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["align.hip", "quant.hip", "gemm.hip", "gemm_w4.hip", "fc1_decode.hip", "down_combine.hip", "combine.hip", "capi.hip"]
# Benchmark-only device-clock marks, a library of their own.
BENCH_SOURCES = ["bench_clock.hip"]
BENCH_LIB = os.path.join(HERE, "libmoebench.so")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know the target feature
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out

    with ThreadPoolExecutor(min(len(SOURCES) + len(BENCH_SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES + BENCH_SOURCES))
    for obj, out in results:
        if verbose and out.strip():
            print(out)
    n = len(SOURCES)
    for lib, objs in ((LIB, results[:n]), (BENCH_LIB, results[n:])):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *[o for o, _ in objs]])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
