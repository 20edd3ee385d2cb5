"""Build the CPU oracle with AddressSanitizer and UBSan (gcc, host code
only) and drive it through random traces, invalid rows and appends."""
import os
import shutil
import subprocess

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           obuild.SRC, os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0")
    proc = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert proc.returncode == 0, proc.stdout + proc.stderr[-2000:]
    assert "ok" in proc.stdout
