"""Host-side preparation of a workload's inputs: its selection trace, the host
rows the trace can read, and the rows appended to a growing context.

Shared by the GPU tests, the benchmark and the oracle-side tests; holds none
of the method's arithmetic.  Host rows of a stream are filled only where the
trace can read them (its selections and resident windows): row p's bytes are
a pure function of (data seed, request, layer, p), so this equals a full fill
on every row that matters.
"""
from __future__ import annotations

import numpy as np

from . import rows as wrows
from .configs import Workload
from .traces import full_trace, multi_query_trace, touched_positions


def make_trace(cfg: Workload, streams=None, queries: int = 1) -> np.ndarray:
    """int32 [steps, layers, B, k] selections; with queries > 1 each row holds
    the queries' selections end to end."""
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
    """Bytes of the row appended at position p of stream (b, l)."""
    return wrows.make_row(cfg.row_elems, p, cfg.data_seed, b, l)
