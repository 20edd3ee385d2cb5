"""Plain float64 sparse-MLA decode attention, for the exactness invariant.

TEST INFRASTRUCTURE ONLY.

The paper listing "HiSparse: Scaling Sparse-Attention Decoding with
Hierarchical KV Cache Management" (Abstract) states that only KV placement
changes, so model outputs are unchanged.  The check built on it: attention of
a query over the rows gathered through the slot map equals attention over the
same positions read straight from the full host history.

One row is a sparse-MLA latent row of 576 values: the first 512 are the
compressed latent (shared by keys and values), the last 64 the rope part of
the key.  For H query heads q[h] (576 values each):

    score[h, i] = scale * sum_e q[h, e] * row_i[e]          (all 576 values)
    w[h, i]     = exp(score[h, i] - max_i score[h, i]) / sum_i (same)
    out[h, :]   = sum_i w[h, i] * row_i[:512]

Computed in float64 from the exact bf16 values, in the order the rows are
given.
"""
from __future__ import annotations

import numpy as np

D_LATENT = 512


def bf16_to_f64(raw: np.ndarray) -> np.ndarray:
    """Decode rows of little-endian bf16 bytes (uint8 [n, 2*d]) to float64 [n, d]."""
    u16 = np.ascontiguousarray(raw).view(np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def mla_decode_attention(q: np.ndarray, rows: np.ndarray, scale: float) -> np.ndarray:
    """q: float64 [H, 576]; rows: float64 [n, 576] in selection order -> [H, 512]."""
    H = q.shape[0]
    n = rows.shape[0]
    out = np.zeros((H, D_LATENT), np.float64)
    if n == 0:
        return out
    for h in range(H):
        score = scale * (rows * q[h][None, :]).sum(axis=1)
        w = np.exp(score - score.max())
        w = w / w.sum()
        out[h] = (w[:, None] * rows[:, :D_LATENT]).sum(axis=0)
    return out


def masked_dense_attention(q: np.ndarray, all_rows: np.ndarray, mask: np.ndarray,
                           scale: float) -> np.ndarray:
    """Attention over the full history in position order, with the positions
    outside ``mask`` excluded (weight exactly 0)."""
    return mla_decode_attention(q, all_rows[mask], scale)


def mla_decode_attention_lse(q: np.ndarray, rows: np.ndarray, scale: float):
    """As mla_decode_attention, also returning lse[h] = log sum_i exp(score[h, i]).
    With no rows the output is 0 and lse is -inf."""
    H = q.shape[0]
    out = np.zeros((H, D_LATENT), np.float64)
    lse = np.full(H, -np.inf)
    if rows.shape[0] == 0:
        return out, lse
    for h in range(H):
        score = scale * (rows * q[h][None, :]).sum(axis=1)
        m = score.max()
        e = np.exp(score - m)
        z = e.sum()
        out[h] = ((e / z)[:, None] * rows[:, :D_LATENT]).sum(axis=0)
        lse[h] = m + np.log(z)
    return out, lse
