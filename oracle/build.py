"""Build the fp64 CPU oracle (test infrastructure) with gcc.

Produces ``oracle/libhalo_ref.so`` from ``oracle/halo_ref.c``.  Plain C, OpenMP
over (batch, head) slices, no fast-math so the arithmetic stays IEEE fp64.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "halo_ref.c")
LIB_PATH = os.path.join(HERE, "libhalo_ref.so")


def build() -> str:
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
