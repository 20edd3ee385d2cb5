"""Seeded selection traces: what a top-k indexer would hand the cache each step.

The pages say the method is indexer-agnostic ([P3] "HiSparse: Scaling
Sparse-Attention Decoding with Hierarchical KV Cache Management", Abstract):
the cache only sees, per layer and step, a set of a few thousand distinct
positions.  Real indexers need trained weights, so a seeded Markov process
stands in for them:

* step 0 draws all k positions from the workload's replacement distribution;
* every later step keeps ``n_keep = floor(carry_pct * k / 100)`` positions, a
  uniform random subset of the previous step's row, and draws ``k - n_keep``
  new positions from the replacement distribution, rejecting any position that
  was selected in the previous step or is already in the new row (so exactly
  ``n_keep`` positions carry over);
* the finished row is put in a seeded random order (a real top-k has no
  meaningful order, and the order decides which miss gets which victim).

Replacement distributions:
  "uniform": uniform over [0, ctx).
  "zipf":    a distance d in {1..ctx} with P(d) proportional to d**-s (a
             truncated Zipf law, sampled by inverse CDF on a float64 table);
             position = ctx - d, so recent positions are favoured.
  "mix":     each new position is, with probability 1/2, uniform over
             [0, ctx - R) and otherwise Zipf distance; a rejected draw is
             redrawn from the same branch.

Several query tokens per step (multi-token prediction, speculative
decoding): query 0 follows the process above with k/Q positions; each other
query keeps a uniform random subset of ``overlap_pct`` percent of query 0's
positions (neighbouring tokens attend to much the same history) and draws the
rest from the replacement distribution, distinct from query 0's row, then is
put in a seeded random order.  The Q rows are laid end to end.

This module holds none of the method's arithmetic.
"""
from __future__ import annotations

import functools

import numpy as np

from .configs import Workload


@functools.lru_cache(maxsize=16)
def _zipf_cdf(ctx: int, s: float) -> np.ndarray:
    d = np.arange(1, ctx + 1, dtype=np.float64)
    w = d ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    return cdf


def _sample_zipf_distance(rng: np.random.Generator, ctx: int, s: float, n: int) -> np.ndarray:
    cdf = _zipf_cdf(ctx, s)
    u = rng.random(n)
    d = np.searchsorted(cdf, u, side="right") + 1
    d = np.minimum(d, ctx)
    return (ctx - d).astype(np.int64)


def _draw_distinct(rng, sampler, n: int, taken: np.ndarray) -> np.ndarray:
    """Draw n positions from ``sampler`` that are not marked in ``taken``.

    Draws are examined in the order they were made; the first occurrence of a
    new position is accepted, later repeats and already-taken positions are
    rejected and replaced by further draws.  Accepted positions are marked.
    Raises ValueError when the distribution leaves too few free positions to
    finish in a bounded number of rounds (a context barely larger than the
    selection, under a distribution concentrated on its taken end).
    """
    out = []
    need = n
    rounds = 0
    while need > 0:
        rounds += 1
        if rounds > 20000:
            raise ValueError(f"could not draw {n} distinct free positions ({need} missing): "
                             "the context is too small for this distribution")
        cand = sampler(max(2 * need, 16))
        _, first = np.unique(cand, return_index=True)
        first.sort()
        cand = cand[first]
        cand = cand[~taken[cand]]
        cand = cand[:need]
        taken[cand] = True
        out.append(cand)
        need -= cand.size
    return np.concatenate(out) if out else np.empty(0, np.int64)


def _new_positions(cfg: Workload, rng, ctx: int, n: int, taken: np.ndarray) -> np.ndarray:
    if cfg.replacement == "uniform":
        return _draw_distinct(rng, lambda m: rng.integers(0, ctx, m), n, taken)
    if cfg.replacement == "zipf":
        return _draw_distinct(rng, lambda m: _sample_zipf_distance(rng, ctx, cfg.zipf_s, m), n, taken)
    if cfg.replacement == "mix":
        n_uni = int(rng.binomial(n, 0.5))
        hi = max(1, ctx - cfg.R)
        a = _draw_distinct(rng, lambda m: rng.integers(0, hi, m), n_uni, taken)
        b = _draw_distinct(rng, lambda m: _sample_zipf_distance(rng, ctx, cfg.zipf_s, m), n - n_uni, taken)
        return np.concatenate([a, b])
    raise ValueError(f"unknown replacement distribution {cfg.replacement!r}")


def stream_seed(cfg: Workload, b: int, l: int) -> np.random.SeedSequence:
    """Trace stream of request b, layer l (layers share one stream when the
    workload shares selections across layers)."""
    if cfg.shared_selection:
        return np.random.SeedSequence([cfg.trace_seed, b])
    return np.random.SeedSequence([cfg.trace_seed, b, l])


def stream_trace(cfg: Workload, b: int, l: int, steps: int | None = None) -> np.ndarray:
    """Selections of one stream: int32 array [steps, k]."""
    steps = cfg.steps if steps is None else steps
    rng = np.random.default_rng(stream_seed(cfg, b, l))
    k = cfg.k
    out = np.empty((steps, k), np.int32)
    prev = None
    taken = np.zeros(cfg.L0 + cfg.growth * max(0, steps - 1) + 1, bool)
    for s in range(steps):
        ctx = cfg.ctx_at(s)
        if k > ctx:
            raise ValueError("k exceeds the context length")
        if prev is None:
            row = _new_positions(cfg, rng, ctx, k, taken)
        else:
            kept = rng.choice(prev, cfg.n_keep, replace=False)
            taken[prev] = True
            new = _new_positions(cfg, rng, ctx, cfg.n_new, taken)
            taken[prev] = False
            row = np.concatenate([kept.astype(np.int64), new])
        row = rng.permutation(row)
        taken[row] = False
        out[s] = row
        prev = row
    return out


def ctx_trace(cfg: Workload, steps: int | None = None) -> np.ndarray:
    steps = cfg.steps if steps is None else steps
    return np.array([cfg.ctx_at(s) for s in range(steps)], np.int64)


def full_trace(cfg: Workload, steps: int | None = None, streams=None) -> np.ndarray:
    """Selections of every stream: int32 [steps, layers, B, k].

    ``streams`` optionally restricts generation to a list of (b, l) pairs; the
    other entries are left as -1 (padding).  Shared-selection workloads
    generate one stream per request and copy it to every layer.
    """
    steps = cfg.steps if steps is None else steps
    out = np.full((steps, cfg.layers, cfg.B, cfg.k), -1, np.int32)
    want = None if streams is None else set(streams)
    cache = {}
    for l in range(cfg.layers):
        for b in range(cfg.B):
            if want is not None and (b, l) not in want:
                continue
            key = (b, 0) if cfg.shared_selection else (b, l)
            if key not in cache:
                cache[key] = stream_trace(cfg, b, l, steps)
            out[:, l, b, :] = cache[key]
    return out


def multi_query_trace(cfg: Workload, queries: int, overlap_pct: int = 75,
                      steps: int | None = None, streams=None) -> np.ndarray:
    """Selections of ``queries`` query tokens per step: int32 [steps, layers,
    B, k], each row the Q query rows of k/Q positions laid end to end."""
    if queries < 1 or cfg.k % queries:
        raise ValueError("k must be a multiple of the number of queries")
    steps = cfg.steps if steps is None else steps
    kq = cfg.k // queries
    n_keep = overlap_pct * kq // 100
    base = full_trace(cfg.scaled(k=kq), steps=steps, streams=streams)   # query 0
    out = np.full((steps, cfg.layers, cfg.B, cfg.k), -1, np.int32)
    want = None if streams is None else set(streams)
    done = {}
    for l in range(cfg.layers):
        for b in range(cfg.B):
            if want is not None and (b, l) not in want:
                continue
            key = (b, 0) if cfg.shared_selection else (b, l)
            if key in done:
                out[:, l, b] = done[key]
                continue
            rows = np.empty((steps, cfg.k), np.int32)
            for st in range(steps):
                ctx = cfg.ctx_at(st)
                row0 = base[st, l, b].astype(np.int64)
                rows[st, :kq] = row0
                for q in range(1, queries):
                    rng = np.random.default_rng(
                        np.random.SeedSequence([cfg.trace_seed, 17, key[0], key[1], st, q]))
                    taken = np.zeros(ctx, bool)
                    taken[row0] = True
                    kept = rng.choice(row0, n_keep, replace=False)
                    new = _new_positions(cfg, rng, ctx, kq - n_keep, taken)
                    rows[st, q * kq:(q + 1) * kq] = rng.permutation(np.concatenate([kept, new]))
            done[key] = rows
            out[:, l, b] = rows
    return out


def touched_positions(trace_bl: np.ndarray, cfg: Workload, steps: int | None = None) -> np.ndarray:
    """Every host row a stream can ever read: its selections plus the resident
    windows of every step (used to fill only those host rows)."""
    steps = trace_bl.shape[0] if steps is None else steps
    pos = [trace_bl[:steps].reshape(-1).astype(np.int64)]
    if cfg.R > 0:
        lo = max(0, cfg.ctx_at(0) - cfg.R)
        pos.append(np.arange(lo, cfg.ctx_at(steps - 1), dtype=np.int64))
    pos = np.concatenate(pos)
    pos = pos[pos >= 0]
    return np.unique(pos)
