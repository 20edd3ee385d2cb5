"""Build the CPU oracle (plain C, gcc).  Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hisparse_oracle.c")
LIB = os.path.join(HERE, "libhisparse_oracle.so")
CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=(), verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
