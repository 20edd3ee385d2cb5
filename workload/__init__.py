"""Seeded synthetic inputs (selection traces and KV rows) shared by the
oracle-side tests and the GPU path's tests and benchmark.  Holds none of the
method's arithmetic."""
from .configs import WORKLOADS, BENCH_WORKLOAD, Workload  # noqa: F401
