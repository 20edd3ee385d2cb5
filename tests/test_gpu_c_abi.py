"""The C ABI from plain C: tests/c_abi_example (built with the library)
replays the hand-derived LRU example through hisparse_create / resolve /
get_status / destroy with hipMalloc'd buffers and checks every step."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_plain_c_caller_replays_the_hand_example():
    binary = os.path.join(HERE, "c_abi_example")
    assert os.path.exists(binary), "tests/c_abi_example is built by __graft_entry__.build()"
    golden = os.path.join(HERE, "golden", "lru_hand_example.txt")
    r = subprocess.run([binary, golden], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "5 steps of the hand example match" in r.stdout
