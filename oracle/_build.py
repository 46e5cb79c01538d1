"""Compiles the CPU oracle (``mlp_oracle.c``) into ``oracle/libmlporacle.so`` with gcc.

Plain -O2 with OpenMP; no tuning flags. Test infrastructure only.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mlp_oracle.c")
LIB_PATH = os.path.join(HERE, "libmlporacle.so")


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle(verbose=True))
