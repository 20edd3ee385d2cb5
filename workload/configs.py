"""The five seeded synthetic workloads the resolve path is tested and measured on.

Each workload is a set of independent *streams*, one per (request, layer): a
stream owns C LRU slots, R resident-window slots and a host history of
``l_cap`` rows.  A row is one token (576 bf16 = 512 latent + 64 rope, the
sparse-MLA row shape) or one 16-token page (Quest-style page granularity).

Sources for the shapes (pages, cited by title and section):
  [P3] "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache
       Management" -- Abstract: a decode step reads a few thousand selected KV
       entries; the selector may be DSA-, NSA- or Quest-style; contexts reach
       far beyond HBM.
  [P2] "Hybrid HiSparse" -- Timeline: the system is evaluated at a full
       1M-token context; cold KV pages live in host memory.
  [P1] "HiSparse" -- Timeline: per-layer independent selections exist
       (absorption layers that each keep their own selection), which rules out
       cross-layer prefetch for them.

This module holds no part of the method's arithmetic: it only names sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

TOKEN_ROW_ELEMS = 576          # 512 latent + 64 rope, bf16
TOKEN_ROW_BYTES = 2 * TOKEN_ROW_ELEMS   # 1152
PAGE_TOKENS = 16
PAGE_ROW_ELEMS = PAGE_TOKENS * TOKEN_ROW_ELEMS  # 9216
PAGE_ROW_BYTES = 2 * PAGE_ROW_ELEMS             # 18432


@dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # requests
    layers: int            # layers, each with its own cache
    L0: int                # context length (rows) at step 0
    growth: int            # rows appended per step (before steps >= 1)
    row_elems: int         # bf16 elements per row
    C: int                 # LRU slots per stream
    R: int                 # resident-window slots per stream
    k: int                 # selections per stream per step
    steps: int
    carry_pct: int         # percent of the previous step's selections kept
    replacement: str       # "uniform" | "mix" | "zipf"
    zipf_s: float = 0.0
    shared_selection: bool = False   # one selection per request used by all layers
    trace_seed: int = 0
    data_seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def row_bytes(self) -> int:
        return 2 * self.row_elems

    @property
    def l_cap(self) -> int:
        """Host-history capacity in rows: the largest context any step sees."""
        return self.L0 + self.growth * max(0, self.steps - 1)

    def ctx_at(self, step: int) -> int:
        return self.L0 + self.growth * step

    @property
    def n_keep(self) -> int:
        """Selections carried over per step: floor(carry_pct * k / 100)."""
        return (self.carry_pct * self.k) // 100

    @property
    def n_new(self) -> int:
        return self.k - self.n_keep

    @property
    def label(self) -> str:
        """Short file-name form of the workload: row kind, requests (x
        layers), context length."""
        kind, _, rest = self.name.partition("_")
        parts = rest.split("_")
        b = parts[0]
        l = parts[1]
        ctx = next(x for x in parts if x.startswith("L") and x[1:2].isdigit())
        return f"{kind}_{b}{'' if l == 'l1' else 'x' + l[1:]}_{ctx}"

    @property
    def streams(self) -> int:
        return self.B * self.layers

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(
        name="tokens_b1_l1_L32k_C4096_k2048",
        B=1, layers=1, L0=32768, growth=0, row_elems=TOKEN_ROW_ELEMS,
        C=4096, R=0, k=2048, steps=8, carry_pct=90, replacement="uniform",
        trace_seed=1001, data_seed=2001,
        description="1 request, 1 layer, L=32768 token rows of 1152 B, C=4096, "
                    "no resident window, k=2048, 8 steps, 90% carry-over, "
                    "uniform replacements"),
    2: Workload(
        name="tokens_b8_l1_L128k_C4096_R128_k2048",
        B=8, layers=1, L0=131072, growth=0, row_elems=TOKEN_ROW_ELEMS,
        C=4096, R=128, k=2048, steps=64, carry_pct=85, replacement="mix",
        zipf_s=1.1, trace_seed=1002, data_seed=2002,
        description="8 requests, 1 layer, L=131072 token rows of 1152 B, C=4096, "
                    "R=128, k=2048, 64 steps, 85% carry-over, replacements half "
                    "uniform over [0,L-R) and half Zipf(1.1) over distance from "
                    "the context end"),
    3: Workload(
        name="tokens_b16_l8_indep_L128k_grow_C6144_R128_k2048",
        B=16, layers=8, L0=131072, growth=1, row_elems=TOKEN_ROW_ELEMS,
        C=6144, R=128, k=2048, steps=32, carry_pct=80, replacement="uniform",
        trace_seed=1003, data_seed=2003,
        description="16 requests x 8 layers with independent per-layer "
                    "selections (DSA-style), L=131072 growing by 1 row per "
                    "step, C=6144, R=128, k=2048, 32 steps, 80% carry-over, "
                    "uniform replacements"),
    4: Workload(
        name="tokens_b16_l8_shared_L256k_C4096_R64_k2048",
        B=16, layers=8, L0=262144, growth=0, row_elems=TOKEN_ROW_ELEMS,
        C=4096, R=64, k=2048, steps=32, carry_pct=75, replacement="zipf",
        zipf_s=1.0, shared_selection=True, trace_seed=1004, data_seed=2004,
        description="16 requests x 8 layers sharing one selection per step, "
                    "L=262144, C=4096 per layer, R=64, k=2048, 32 steps, 75% "
                    "carry-over, Zipf(1.0) recency-skewed replacements; the "
                    "next layer is prefetched on a second stream"),
    5: Workload(
        name="pages_b4_l4_L1M_C512_R1_k128",
        B=4, layers=4, L0=65536, growth=0, row_elems=PAGE_ROW_ELEMS,
        C=512, R=1, k=128, steps=64, carry_pct=70, replacement="uniform",
        trace_seed=1005, data_seed=2005,
        description="4 requests x 4 layers, 1M tokens as 65536 pages of 16 "
                    "rows (18432 B per page), k=128 pages, C=512 page slots, "
                    "R=1 page, 64 steps, 70% carry-over, uniform page "
                    "replacements; also run with copies suppressed"),
}

# The workload the headline throughput is quoted on (fits one GPU).
BENCH_WORKLOAD = 4
