"""Build the C oracle into oracle/libss_oracle.so (test infrastructure).

    python oracle/build.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libss_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ss_oracle.c")
    tmp = LIB + ".tmp"
    # No fast-math and no FMA contraction: the oracle is the plain loop.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-Wno-unused-parameter", "-Wno-missing-field-initializers",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
