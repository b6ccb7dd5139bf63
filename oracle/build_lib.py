"""Build liboracle.so from oracle.c with the host C compiler (test infrastructure).

Plain ISO C11 in double precision: no fast-math, no FMA contraction, so every
rounding is the one the source states.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, os.path.join(HERE, "oracle.c"),
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
