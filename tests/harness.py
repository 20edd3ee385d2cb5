"""Shared test plumbing: seeded workloads -> host rows -> oracle streams.

The oracle and the GPU library read the very same host buffers; the host
rows, traces and appended rows come from workload.prepare.
"""
from __future__ import annotations

from oracle.oracle import OracleStream, resolve_multi
from workload.configs import Workload
from workload.prepare import appended_row, fill_host, make_trace  # noqa: F401


def small_variant(cfg: Workload, **kw) -> Workload:
    """A reduced copy of a workload that keeps its structure (shared or
    independent selections, growth, window, row size, carry-over)."""
    return cfg.scaled(**kw)


class OracleRun:
    """Oracle streams for a set of (b, l) pairs of a workload."""

    def __init__(self, cfg: Workload, streams, host_of=None, with_data=True):
        self.cfg = cfg
        self.streams = list(streams)
        self.st = {}
        for (b, l) in self.streams:
            host = host_of(b, l) if host_of is not None else None
            self.st[(b, l)] = OracleStream(cfg.C, cfg.R, cfg.l_cap, cfg.row_bytes,
                                           host=host, with_data=with_data)
            self.st[(b, l)].seed_window(cfg.ctx_at(0))

    def append(self, step: int):
        """Grow every stream's context by one row before ``step``."""
        p = self.cfg.ctx_at(step) - 1
        for (b, l), st in self.st.items():
            st.append(appended_row(self.cfg, b, l, p), p)

    def step(self, s: int, trace: np.ndarray, no_io: bool = False, queries: int = 1):
        """One step on every stream; with queries > 1 each trace row holds the
        queries' selections end to end and `out` comes back flattened."""
        ctx = self.cfg.ctx_at(s)
        if queries > 1:
            res = {}
            for (b, l), st in self.st.items():
                r = resolve_multi(st, trace[s, l, b].reshape(queries, -1), ctx, no_io=no_io)
                r.out = r.out.reshape(-1)
                res[(b, l)] = r
            return res
        return {(b, l): st.resolve(trace[s, l, b], ctx, no_io=no_io)
                for (b, l), st in self.st.items()}
