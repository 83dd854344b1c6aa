"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "gemm_oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    # -O2, no fast-math: the float64 sums must stay plain IEEE arithmetic.
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
