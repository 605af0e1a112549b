"""Builds libmoe_dispatch.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep float arithmetic exactly as written (no contraction of separate multiply/add; every
    # fused multiply-add in the kernels is an explicit fma)
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def library_path() -> str:
    return os.path.join(HERE, "libmoe_dispatch.so")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
