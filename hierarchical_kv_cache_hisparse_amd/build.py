"""Build libhisparse.so for gfx950 with hipcc (in-tree, next to the binding)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhisparse.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed FP32 instructions are switched off.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = [("hisparse_kernels.hip", True), ("hisparse_mla.hip", True), ("hisparse_topk.hip", True),
           ("hisparse_noalloc.hip", True), ("hisparse_runtime.cpp", False)]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    for name, device in SOURCES:
        src = os.path.join(CSRC, name)
        obj = os.path.join(OBJDIR, name + ".o")
        cmd = [HIPCC, *COMMON, *(DEVICE if device else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]),
               "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
