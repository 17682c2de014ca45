"""Compile the fp64 oracle (plain C) into oracle/libsmla_ref.so with gcc.

Strict IEEE fp64: no fast-math, no FMA contraction, so the oracle's rounding
is the straightforward left-to-right evaluation written in smla_ref.c.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "smla_ref.c")
OUT = os.path.join(_HERE, "libsmla_ref.so")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
