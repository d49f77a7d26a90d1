"""Compile the CPU oracle (test infrastructure) into ``oracle/liboracle.so``.

gcc, -O2, IEEE semantics: no -ffast-math (it would turn on flush-to-zero on
x86) and no floating-point contraction (no fused multiply-add)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gcq_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
