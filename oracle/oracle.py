"""Python face of the CPU oracle (hisparse_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library or its binding.

``OracleStream`` owns one stream's state -- one (request, layer) cache -- as
numpy arrays and calls the C oracle to resolve a step.  See the C file for the
method's statement and the readings it takes where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

STATUS_SEL_RANGE = 1
STATUS_SEL_DUP = 2
STATUS_CTX_RANGE = 4
STATUS_CAPACITY = 8
FLAG_NO_IO = 1

COUNTER_NAMES = ("n_pad", "n_res", "n_hit", "n_miss", "n_evict", "bytes")


class _Stream(ctypes.Structure):
    _fields_ = [
        ("C", ctypes.c_int32),
        ("R", ctypes.c_int32),
        ("l_cap", ctypes.c_int64),
        ("row_bytes", ctypes.c_int64),
        ("pos2slot", ctypes.c_void_p),
        ("slot2pos", ctypes.c_void_p),
        ("last_use", ctypes.c_void_p),
        ("t", ctypes.c_void_p),
        ("slots", ctypes.c_void_p),
        ("host", ctypes.c_void_p),
    ]


_lib = None


def load(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} missing: run `python -m oracle.build`")
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    lib.hso_resolve.argtypes = [P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, P, P, P, P]
    lib.hso_resolve.restype = ctypes.c_uint32
    lib.hso_seed_window.argtypes = [P, ctypes.c_int64]
    lib.hso_seed_window.restype = ctypes.c_int
    lib.hso_append.argtypes = [P, P, ctypes.c_int64]
    lib.hso_append.restype = ctypes.c_int
    return lib


@dataclass
class StepResult:
    status: int
    out: np.ndarray          # int32 [k]
    log_slot: np.ndarray     # int32 [n_miss]
    log_old: np.ndarray      # int32 [n_miss]
    counters: dict


class OracleStream:
    """State of one (request, layer) cache: C LRU slots + R resident slots.

    ``host`` is the stream's host history, uint8 [l_cap, row_bytes]; pass
    ``with_data=False`` to simulate metadata only (no slot bytes).
    """

    def __init__(self, C: int, R: int, l_cap: int, row_bytes: int,
                 host: np.ndarray | None = None, with_data: bool = True, lib=None):
        self.lib = lib or load()
        self.C, self.R, self.l_cap, self.row_bytes = C, R, l_cap, row_bytes
        self.pos2slot = np.full(l_cap, -1, np.int32)
        self.slot2pos = np.full(C, -1, np.int32)
        self.last_use = np.zeros(C, np.int32)
        self.t = np.zeros(1, np.int32)
        if host is not None:
            if host.dtype != np.uint8 or host.shape != (l_cap, row_bytes) or not host.flags.c_contiguous:
                raise ValueError("host must be a C-contiguous uint8 [l_cap, row_bytes] array")
        self.host = host
        self.slots = np.zeros((C + R, row_bytes), np.uint8) if (with_data and host is not None) else None
        self._st = _Stream(C, R, l_cap, row_bytes,
                           self.pos2slot.ctypes.data, self.slot2pos.ctypes.data,
                           self.last_use.ctypes.data, self.t.ctypes.data,
                           None if self.slots is None else self.slots.ctypes.data,
                           None if host is None else host.ctypes.data)
        self._scratch_k = 0

    def seed_window(self, ctx: int) -> None:
        if self.slots is None:
            return
        if self.lib.hso_seed_window(ctypes.byref(self._st), ctx) != 0:
            raise ValueError("seed_window: bad context length")

    def append(self, row: np.ndarray, ctx: int) -> None:
        row = np.ascontiguousarray(row, dtype=np.uint8)
        if row.size != self.row_bytes:
            raise ValueError("row has the wrong size")
        if self.lib.hso_append(ctypes.byref(self._st), row.ctypes.data, ctx) != 0:
            raise ValueError("append: position outside the host history")

    def resolve(self, sel, ctx: int, no_io: bool = False) -> StepResult:
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        k = sel.size
        out = np.empty(k, np.int32)
        log_slot = np.empty(max(k, 1), np.int32)
        log_old = np.empty(max(k, 1), np.int32)
        cnt = np.zeros(6, np.int64)
        status = self.lib.hso_resolve(ctypes.byref(self._st), sel.ctypes.data, k, ctx,
                                      FLAG_NO_IO if no_io else 0, out.ctypes.data,
                                      log_slot.ctypes.data, log_old.ctypes.data, cnt.ctypes.data)
        m = int(cnt[3]) if status == 0 else 0
        return StepResult(int(status), out, log_slot[:m].copy(), log_old[:m].copy(),
                          dict(zip(COUNTER_NAMES, (int(x) for x in cnt))))

    # -- snapshot / restore of the whole state ------------------------------
    def snapshot(self) -> dict:
        snap = {"pos2slot": self.pos2slot.copy(), "slot2pos": self.slot2pos.copy(),
                "last_use": self.last_use.copy(), "t": self.t.copy()}
        if self.slots is not None:
            snap["slots"] = self.slots.copy()
        return snap

    def restore(self, snap: dict) -> None:
        self.pos2slot[:] = snap["pos2slot"]
        self.slot2pos[:] = snap["slot2pos"]
        self.last_use[:] = snap["last_use"]
        self.t[:] = snap["t"]
        if self.slots is not None:
            self.slots[:] = snap["slots"]



def resolve_multi(stream: OracleStream, sel, ctx: int, no_io: bool = False) -> StepResult:
    """Selections of several query tokens of one request, resolved in one step.

    Reading: the pages list multi-token prediction only as a feature the
    method stays compatible with ("Hybrid HiSparse", Timeline).  Every query
    token of the step attends through the same cache, so the cache has to hold
    the union of their selections at once; the step is therefore one
    resolution of that union, which is one clock tick for the stream.  The
    union is written in first-occurrence order over the entries (query-major,
    then index) and padded with -1 to the Q*k entries of the call, so that a
    position that misses is fetched once and the j-th distinct miss takes the
    j-th victim.  Every entry is then served by its position's slot; padding
    stays -1.  The counters and the eviction log are those of the union row.
    A rejected union (any entry outside [-1, ctx), or a bad ctx) serves -1
    everywhere and leaves the stream untouched, as the single-query step does.

    sel: int [Q, k].  Returns a StepResult whose `out` is int32 [Q, k].
    """
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    if sel.ndim != 2:
        raise ValueError("sel must be [queries, k]")
    Q, k = sel.shape
    flat = sel.reshape(-1).tolist()
    union = np.full(Q * k, -1, np.int32)
    first = {}
    for p in flat:
        if p != -1 and p not in first:
            first[p] = len(first)
            union[first[p]] = p
    r = stream.resolve(union, ctx, no_io=no_io)
    out = np.array([-1 if p == -1 else int(r.out[first[p]]) for p in flat], np.int32)
    return StepResult(r.status, out.reshape(Q, k), r.log_slot, r.log_old, r.counters)
