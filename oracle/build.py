"""Builds the CPU oracle shared library (plain C, gcc). Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")


def library_path() -> str:
    return os.path.join(HERE, "libmoe_oracle.so")


def build() -> str:
    """Compile moe_oracle.c with no FP contraction and no fast-math; returns the .so path."""
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
