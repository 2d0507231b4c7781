"""Build liblayeradam.so (the HIP library behind include/layeradam.h) in-tree.

    python -m optimizer_step_layeradam_amd.build

Compiles csrc/*.hip and csrc/*.cpp with hipcc for gfx950 into
optimizer_step_layeradam_amd/liblayeradam.so. Always recompiles.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "liblayeradam.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # one IEEE rounding per operation: no contraction into fused multiply-add
    "-ffp-contract=off",
    # no packed FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build(verbose: bool = False, out: str = LIB_PATH, extra=()) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), "-o", out + ".tmp", *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
