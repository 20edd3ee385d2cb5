"""Two-tier (host + GPU) KV cache for top-k sparse-attention decoding on AMD
MI355X: per-layer selection resolution (hit detection, LRU replacement,
host-to-device miss fetch) in hand-written gfx950 HIP kernels behind a C ABI
(include/hisparse.h).  ``binding`` is the thin ctypes layer over it; the
library is loaded on first use and its absence is an error, never a
fallback."""
from . import binding  # noqa: F401
from .binding import *  # noqa: F401,F403
