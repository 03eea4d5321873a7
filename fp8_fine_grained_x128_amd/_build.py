"""Compile the HIP sources under csrc/ into the in-tree ``libfp8q.so``.

Every source is compiled for gfx950 with hipcc, without fast-math and without
floating-point contraction (the quantizers must reproduce exact fp32 operation
sequences), and with packed FP32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["quantize.hip", "gemm.hip", "transpose.hip", "fp8q_api.hip", "clock_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-fast-math", "-Wall", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source additions.  The GEMM kernels are scheduled with LLVM's iterative
# ILP strategy: on gfx950 it fits the fprop strip kernel in 255 VGPRs without
# spills (the default strategy spills 2) and measured 1.5 % faster on the
# plain GEMM and 3 % on the grouped GEMM, with bit-identical outputs.
SOURCE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    """Compile every source and link libfp8q.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
