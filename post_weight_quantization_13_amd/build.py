"""Builds libgptq.so (every HIP source under csrc/) for gfx950 with hipcc.

Usage: python -m post_weight_quantization_13_amd.build   (or build() from Python).
Objects go to _build/ next to this file; the library is written in-tree so the
package loads it from its own directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgptq.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # hipcc -O3 forms packed fp32 instructions from scalar code on its own; they
    # are kept out of every kernel here.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Register-resident arrays (the 64-row factorization keeps a row per lane)
    # need their loops fully unrolled; the default size limit on explicitly
    # unrolled loops would leave some rolled and move the arrays to scratch.
    "-mllvm", "-pragma-unroll-threshold=500000",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libgptq)")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
