"""Compile the oracle's C source into oracle/libq4_0_oracle.so with gcc.

Plain -O2, no fast-math, no vector intrinsics: the oracle must stay an
obviously correct reading of the definition, not a tuned kernel.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_0_oracle.c")
LIB = os.path.join(HERE, "libq4_0_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           "-o", lib + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
