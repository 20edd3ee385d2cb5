"""Seeded synthetic indexer scores: one float32 score per position (a token
for DSA-style selection, a page for Quest-style selection), standing in for a
trained indexer's output.

Scores of request b, layer l at step s:

    score[p] = base[p] + drift * noise_s[p]

base is N(0,1) per (seed, request, layer), fixed over the steps, and noise_s
is N(0,1) per (seed, request, layer, step), so consecutive steps select
largely the same positions (decode queries change slowly).  Options:

  * ``ties``: scores rounded to bfloat16 precision (round to nearest even),
    so equal scores occur at the selection boundary;
  * ``specials``: a few positions get -inf, +0.0 and -0.0.

Generated with numpy's PCG64 through SeedSequence([seed, request, layer]) and
([seed, request, layer, step + 1]).  This module holds none of the method's
arithmetic.
"""
from __future__ import annotations

import numpy as np


def _round_bf16(x: np.ndarray) -> np.ndarray:
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def score_row(n: int, seed: int, b: int, l: int, step: int, drift: float = 0.35,
              ties: bool = False, specials: bool = False) -> np.ndarray:
    base = np.random.default_rng(np.random.SeedSequence([seed, b, l])).standard_normal(
        n, dtype=np.float32)
    rng = np.random.default_rng(np.random.SeedSequence([seed, b, l, step + 1]))
    row = base + np.float32(drift) * rng.standard_normal(n, dtype=np.float32)
    if ties:
        row = _round_bf16(row)
    if specials and n >= 8:
        idx = rng.choice(n, 6, replace=False)
        row[idx[:2]] = -np.inf
        row[idx[2:4]] = np.float32(0.0)
        row[idx[4:]] = np.float32(-0.0)
    return row.astype(np.float32)


def score_rows(B: int, n: int, seed: int, l: int, step: int, **kw) -> np.ndarray:
    """float32 [B, n]."""
    return np.stack([score_row(n, seed, b, l, step, **kw) for b in range(B)])
