"""Build the seeded row generator (plain C, gcc, OpenMP)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rowgen.c")
LIB = os.path.join(HERE, "libhsrowgen.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
