"""Seeded KV row bytes (N(0,1) -> bf16), filled by the C generator in rowgen.c.

Row p of stream (request b, layer l) is a pure function of (data seed, b, l,
p), so filling only the rows a trace can touch gives the same bytes as
filling all of them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(
                f"{_build.LIB} is missing: run `python -m workload.build` "
                "(or __graft_entry__.build())")
        lib = ctypes.CDLL(_build.LIB)
        i64, u32, p = ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
        lib.hsw_fill_range.argtypes = [p, i64, i64, i64, u32, u32, u32]
        lib.hsw_fill_rows.argtypes = [p, i64, p, i64, u32, u32, u32]
        lib.hsw_make_row.argtypes = [p, i64, i64, u32, u32, u32]
        for f in (lib.hsw_fill_range, lib.hsw_fill_rows, lib.hsw_make_row):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check_rows(host: np.ndarray, row_elems: int):
    if host.dtype != np.uint8 or host.ndim != 2 or host.shape[1] != 2 * row_elems:
        raise ValueError("host rows must be a uint8 array [rows, 2*row_elems]")
    if not host.flags.c_contiguous:
        raise ValueError("host rows must be C-contiguous")


def fill_range(host: np.ndarray, row_elems: int, p0: int, n: int, seed: int, b: int, l: int):
    """Fill rows [p0, p0+n) of ``host`` (uint8 [rows, row_bytes])."""
    _check_rows(host, row_elems)
    if p0 < 0 or p0 + n > host.shape[0]:
        raise ValueError("row range outside the host buffer")
    rc = _load().hsw_fill_range(host.ctypes.data, row_elems, p0, n, seed, b, l)
    if rc != 0:
        raise ValueError("hsw_fill_range rejected its arguments")


def fill_rows(host: np.ndarray, row_elems: int, rows, seed: int, b: int, l: int):
    """Fill the listed rows of ``host`` (uint8 [rows, row_bytes])."""
    _check_rows(host, row_elems)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= host.shape[0]):
        raise ValueError("row index outside the host buffer")
    rc = _load().hsw_fill_rows(host.ctypes.data, row_elems, rows.ctypes.data, rows.size,
                               seed, b, l)
    if rc != 0:
        raise ValueError("hsw_fill_rows rejected its arguments")


def make_row(row_elems: int, p: int, seed: int, b: int, l: int) -> np.ndarray:
    """Bytes of row p of stream (b, l) as uint8 [row_bytes]."""
    out = np.empty(2 * row_elems, np.uint8)
    rc = _load().hsw_make_row(out.ctypes.data, row_elems, p, seed, b, l)
    if rc != 0:
        raise ValueError("hsw_make_row rejected its arguments")
    return out


def bf16_bytes_to_f64(raw: np.ndarray) -> np.ndarray:
    """Decode little-endian bf16 bytes to float64 (exact)."""
    u16 = np.ascontiguousarray(raw).view(np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_queries(B: int, H: int, seed: int, layer: int) -> np.ndarray:
    """Seeded query heads for sparse-MLA decode: bf16 bytes uint8 [B, H, 1152]
    (576 values per head, N(0,1) like the rows, from their own seed)."""
    out = np.empty((B, H, 1152), np.uint8)
    for b in range(B):
        for h in range(H):
            out[b, h] = make_row(576, h, seed, b, layer)
    return out
