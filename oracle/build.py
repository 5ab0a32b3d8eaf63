"""ORACLE build step (test infrastructure): compile the oracle's C part with gcc.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
what this builds.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "router_logits.c")
LIB = os.path.join(HERE, "liboracle_router.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile liboracle_router.so next to its source (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only if the shared object is missing."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
