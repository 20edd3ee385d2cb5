"""Plain top-k selection over per-position indexer scores.

TEST INFRASTRUCTURE ONLY.

The method takes, per layer and step, the positions a top-k indexer picked
and is agnostic to the indexer ("HiSparse: Scaling Sparse-Attention Decoding
with Hierarchical KV Cache Management", Abstract: sparse attention with top-k
selection; "Hybrid HiSparse", Timeline: token- and page-granular selection).
This is the step that produces those positions from one score per position
(a token for DSA-style selection, a page for Quest-style selection).

Readings where the pages are silent:
  * eligible positions are [0, ctx); scores are finite or infinite, never NaN;
  * the k positions with the largest scores are chosen; equal scores are
    broken by the lower position; -0.0 and +0.0 are equal scores;
  * the result lists the chosen positions in ascending position order (the
    pages give a selection no order), padded with -1 to k when ctx < k.

The definition is written out directly: order the eligible positions by
(score descending, position ascending) with a library sort, keep the first k.
"""
from __future__ import annotations

import numpy as np


def topk_select(scores, ctx: int, k: int) -> np.ndarray:
    """Top-k of scores[0:ctx] (float32 or float64): int32 [k], ascending
    positions, -1 padded."""
    if k < 1:
        raise ValueError("k must be >= 1")
    s = np.asarray(scores, dtype=np.float64)[:ctx]
    if ctx < 0 or s.size != ctx:
        raise ValueError("ctx outside the score row")
    if np.isnan(s).any():
        raise ValueError("NaN score")
    pos = np.arange(ctx)
    # np.lexsort: the last key is the primary one; float comparisons treat
    # -0.0 and +0.0 as equal, so such ties fall to the position key.
    order = np.lexsort((pos, -s))
    chosen = np.sort(order[:k])
    out = np.full(k, -1, np.int32)
    out[:chosen.size] = chosen
    return out


def topk_rows(scores2d, ctx_len, k: int) -> np.ndarray:
    """topk_select for every row of a [B, N] score array: int32 [B, k]."""
    return np.stack([topk_select(scores2d[b], int(ctx_len[b]), k)
                     for b in range(len(ctx_len))])
