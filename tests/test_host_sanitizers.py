"""The C runtime's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The runtime (argument validation, layout and workspace arithmetic, NUMA
placement, error strings) is rebuilt with both sanitizers on its host code
and linked with the already-built kernel objects; the host-only ABI tests
then run against that library in a child process with the sanitizer
runtime preloaded, so any out-of-bounds access, use after free or undefined
operation on those paths aborts the run.  No GPU is needed or touched."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_hisparse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL_OBJS = [os.path.join(ROOT, "_build", n + ".o")
               for n in ("hisparse_kernels.hip", "hisparse_mla.hip", "hisparse_topk.hip",
                         "hisparse_noalloc.hip")]
# each -fsanitize applies to host code only
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]

PLUGIN = '''import os
from hierarchical_kv_cache_hisparse_amd import binding as hb
hb.LIB_PATH = os.environ["HISPARSE_TEST_LIB"]
'''


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_runtime_host_code_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or rt is None or not all(map(os.path.exists, KERNEL_OBJS)):
        pytest.skip("needs hipcc, the clang sanitizer runtime and a built library (_build/)")
    if os.environ.get("LD_PRELOAD") or os.path.exists("/etc/ld.so.preload"):
        # the sanitizer runtime has to be the first library loaded; an
        # environment that already preloads one is left as it is
        pytest.skip("the environment already preloads a library")
    obj = str(tmp_path / "hisparse_runtime_san.o")
    lib = str(tmp_path / "libhisparse_san.so")
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"-I{ROOT}/include", f"-I{CSRC}",
                    "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SANITIZE,
                    "-c", os.path.join(CSRC, "hisparse_runtime.cpp"), "-o", obj], check=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", *SANITIZE, *KERNEL_OBJS, obj,
                    "-o", lib], check=True)
    (tmp_path / "san_plugin.py").write_text(PLUGIN)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HISPARSE_TEST_LIB": lib,
        "PYTHONPATH": os.pathsep.join([str(tmp_path), ROOT, env.get("PYTHONPATH", "")]),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "san_plugin", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
