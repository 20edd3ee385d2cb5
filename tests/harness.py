"""Shared test plumbing: seeded workloads -> host rows -> oracle streams.

Host rows of a stream are filled only where the trace can read them (its
selections and resident windows); row p's bytes are a pure function of
(data seed, request, layer, p), so this equals a full fill on every row that
matters.  The oracle and the GPU library read the very same host buffers.
"""
from __future__ import annotations

import numpy as np

from oracle.oracle import OracleStream, resolve_multi
from workload import rows as wrows
from workload.configs import Workload
from workload.traces import full_trace, multi_query_trace, touched_positions


def small_variant(cfg: Workload, **kw) -> Workload:
    """A reduced copy of a workload that keeps its structure (shared or
    independent selections, growth, window, row size, carry-over)."""
    return cfg.scaled(**kw)


def make_trace(cfg: Workload, streams=None, queries: int = 1) -> np.ndarray:
    if queries > 1:
        return multi_query_trace(cfg, queries, streams=streams)
    return full_trace(cfg, streams=streams)


def fill_host(cfg: Workload, host_of, trace: np.ndarray, streams):
    """Fill each stream's host rows that the trace can touch.

    host_of(b, l) -> uint8 [l_cap, row_bytes] array (numpy or pinned view).
    Appended rows (growth) are written later, at append time.
    """
    for (b, l) in streams:
        pos = touched_positions(trace[:, l, b, :], cfg)
        pos = pos[pos < cfg.L0]
        wrows.fill_rows(host_of(b, l), cfg.row_elems, pos, cfg.data_seed, b, l)


def appended_row(cfg: Workload, b: int, l: int, p: int) -> np.ndarray:
    return wrows.make_row(cfg.row_elems, p, cfg.data_seed, b, l)


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
