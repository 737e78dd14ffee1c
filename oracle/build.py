"""Build the CPU oracle (test infrastructure) into oracle/libgqref.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgqref.so")
SRC = os.path.join(HERE, "gqref.c")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def needs_build() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(os.path.join(HERE, f)) > t
               for f in ("gqref.c", "gqref.h"))


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
