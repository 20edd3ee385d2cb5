"""Build tests/c_abi_example (a plain C caller of libhisparse) next to its
source; called by the repository's build step after the library is built."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BINARY = os.path.join(HERE, "c_abi_example")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", os.path.join(HERE, "c_abi_example.c"),
           "-o", BINARY + ".tmp",
           f"-L{ROOT}/hierarchical_kv_cache_hisparse_amd", "-lhisparse",
           f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../hierarchical_kv_cache_hisparse_amd", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY
