"""The CPU oracle against an independent brute-force recency-list simulator
on tiny traces (no GPU)."""
from tests import pins


def test_bruteforce_random_traces():
    pins.check_bruteforce_random(n_traces=400)


def test_bruteforce_exhaustive_tiny():
    pins.check_bruteforce_exhaustive()


def test_data_invariants_small():
    pins.check_data_invariants()
