"""Builds the in-tree HIP library ``kv_quantization_tile_amd/libhq.so`` for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhq.so")
SOURCES = ["hq_kernels.hip", "hq_api.hip", "hq_rotate.hip", "hq_srft.hip"]

# Floating-point flags: every binary32 operation that decides an integer code must be rounded
# exactly once in program order (no contraction into FMA, no fast-math, denormals kept, correctly
# rounded division and square root), so that the kernels reproduce the CPU oracle bit for bit.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # workgroup reductions through LDS atomics at a uniform address become DPP reductions instead
    # of a per-lane read-back loop
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc"] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libhq.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
