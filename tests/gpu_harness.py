"""GPU-side test plumbing: one libhisparse instance driven through the C ABI
next to the CPU oracle on the same host buffers, with state read-back and
element-by-element comparison.  Imported only by GPU tests and the smoke
check.
"""
from __future__ import annotations

import numpy as np

from hierarchical_kv_cache_hisparse_amd import binding as hb
from hierarchical_kv_cache_hisparse_amd.instance import GpuInstance, host_view  # noqa: F401
from tests.harness import OracleRun, appended_row, fill_host, make_trace
from workload import rows as wrows
from workload.configs import Workload


class LockstepRun:
    """A workload run on the GPU next to the oracle (on a subset of streams).

    queries > 1: every row holds that many query tokens' selections end to
    end (k/queries each) and the steps go through hisparse_resolve_multi.
    """

    def __init__(self, cfg: Workload, oracle_streams=None, flags: int = 0,
                 host_flags: int = hb.HISPARSE_HOST_COHERENT, fill_all=False, queries: int = 1):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.queries = queries
        all_streams = [(b, l) for b in range(cfg.B) for l in range(cfg.layers)]
        self.oracle_streams = all_streams if oracle_streams is None else list(oracle_streams)
        self.trace = make_trace(cfg, queries=queries)
        self.gpu = GpuInstance(cfg, flags=flags, host_flags=host_flags)
        if fill_all:
            for (b, l) in all_streams:
                wrows.fill_range(self.gpu.host(b, l), cfg.row_elems, 0, cfg.L0, cfg.data_seed, b, l)
        else:
            fill_host(cfg, self.gpu.host, self.trace, all_streams)
        self.no_io = bool(flags & hb.HISPARSE_NO_IO)
        self.oracle = OracleRun(cfg, self.oracle_streams, host_of=self.gpu.host,
                                with_data=not self.no_io)
        dev = self.gpu.device
        self.sel_dev = torch.from_numpy(self.trace).to(dev)            # [S, L, B, k]
        ctx = np.array([[cfg.ctx_at(s)] * cfg.B for s in range(cfg.steps)], np.int32)
        self.ctx_dev = torch.from_numpy(ctx).to(dev)                    # [S, B]
        self.out_dev = torch.full((cfg.layers, cfg.B, cfg.k), -7, dtype=torch.int32, device=dev)
        self.pos_dev = torch.from_numpy(
            np.array([[cfg.ctx_at(s) - 1] * cfg.B for s in range(cfg.steps)], np.int32)).to(dev)
        hb.hisparse_load_window(self.gpu.h, self.gpu.stream, -1, self.ctx_dev[0].data_ptr())
        torch.cuda.synchronize()

    def append_rows(self, s: int):
        """Grow every stream by one row before step s (host history + ring)."""
        cfg, torch = self.cfg, self.torch
        p = cfg.ctx_at(s) - 1
        for l in range(cfg.layers):
            rows = np.stack([appended_row(cfg, b, l, p) for b in range(cfg.B)])
            rows_dev = torch.from_numpy(rows).to(self.gpu.device)
            hb.hisparse_append(self.gpu.h, self.gpu.stream, l, rows_dev.data_ptr(),
                               self.pos_dev[s].data_ptr())
            torch.cuda.synchronize()
        self.oracle.append(s)

    def append_and_step(self, s: int):
        """Step s of a growing workload through hisparse_append_resolve (or its
        multi-query form): every layer's new row and its resolution in one
        call."""
        cfg, torch = self.cfg, self.torch
        p = cfg.ctx_at(s) - 1
        for l in range(cfg.layers):
            rows = np.stack([appended_row(cfg, b, l, p) for b in range(cfg.B)])
            rows_dev = torch.from_numpy(rows).to(self.gpu.device)
            if self.queries > 1:
                hb.hisparse_append_resolve_multi(
                    self.gpu.h, self.gpu.stream, l, rows_dev.data_ptr(), self.pos_dev[s].data_ptr(),
                    self.sel_dev[s, l].data_ptr(), self.queries, cfg.k // self.queries,
                    self.ctx_dev[s].data_ptr(), self.out_dev[l].data_ptr())
            else:
                hb.hisparse_append_resolve(self.gpu.h, self.gpu.stream, l, rows_dev.data_ptr(),
                                           self.pos_dev[s].data_ptr(),
                                           self.sel_dev[s, l].data_ptr(),
                                           self.ctx_dev[s].data_ptr(), self.out_dev[l].data_ptr())
            torch.cuda.synchronize()
        self.oracle.append(s)

    def gpu_step(self, s: int, layers=None):
        layers = range(self.cfg.layers) if layers is None else layers
        for l in layers:
            if self.queries > 1:
                hb.hisparse_resolve_multi(self.gpu.h, self.gpu.stream,
                                          self.sel_dev[s, l].data_ptr(), self.queries,
                                          self.cfg.k // self.queries, self.ctx_dev[s].data_ptr(),
                                          l, self.out_dev[l].data_ptr())
            else:
                hb.hisparse_resolve(self.gpu.h, self.gpu.stream, self.sel_dev[s, l].data_ptr(),
                                    self.ctx_dev[s].data_ptr(), l, self.out_dev[l].data_ptr())

    def prefetch_step(self, s: int, main: int, side: int, sel=None, ctx=None, out=None,
                      direct=True):
        """Step s with the layer-wise prefetch schedule of shared selections:
        resolve layer 0 on `main`; then for every layer l, prefetch layer l+1
        on `side` (forked from `main` after layer l's call) and resolve layer
        l+1 on `main`, which joins the prefetch.  sel / ctx / out default to
        this run's buffers for step s (a graph passes fixed buffers).  direct:
        the prefetch writes the layer's slot-map buffer itself (the join is an
        event wait); else it writes the library's own buffer and the join
        copies it."""
        sel = self.sel_dev[s] if sel is None else sel
        ctx = self.ctx_dev[s] if ctx is None else ctx
        out = self.out_dev if out is None else out
        h = self.gpu.h
        hb.hisparse_resolve(h, main, sel[0].data_ptr(), ctx.data_ptr(), 0, out[0].data_ptr())
        for l in range(self.cfg.layers - 1):
            hb.hisparse_prefetch(h, main, side, sel[l + 1].data_ptr(), ctx.data_ptr(), l + 1,
                                 out[l + 1].data_ptr() if direct else 0)
            hb.hisparse_resolve(h, main, sel[l + 1].data_ptr(), ctx.data_ptr(), l + 1,
                                out[l + 1].data_ptr())

    def prefetch_ahead_step(self, s: int, main: int, sides, sel=None, ctx=None):
        """Step s with two layers in flight: layer 0 resolved on `main`, layer 1
        prefetched; then before each layer l is joined, layer l+1 is prefetched
        on the other side stream, so its launch runs while layer l's prefetch
        still does.  Every prefetch writes the layer's slot-map buffer itself."""
        sel = self.sel_dev[s] if sel is None else sel
        ctx = self.ctx_dev[s] if ctx is None else ctx
        out = self.out_dev
        h, L = self.gpu.h, self.cfg.layers
        hb.hisparse_resolve(h, main, sel[0].data_ptr(), ctx.data_ptr(), 0, out[0].data_ptr())
        if L > 1:
            hb.hisparse_prefetch(h, main, sides[1 % 2], sel[1].data_ptr(), ctx.data_ptr(), 1,
                                 out[1].data_ptr())
        for l in range(1, L):
            if l + 1 < L:
                hb.hisparse_prefetch(h, main, sides[(l + 1) % 2], sel[l + 1].data_ptr(),
                                     ctx.data_ptr(), l + 1, out[l + 1].data_ptr())
            hb.hisparse_resolve(h, main, sel[l].data_ptr(), ctx.data_ptr(), l, out[l].data_ptr())

    def oracle_step(self, s: int):
        return self.oracle.step(s, self.trace, no_io=self.no_io, queries=self.queries)

    def compare_step(self, s: int, res, full_state=True, contents=True, host_rows=True,
                     full_streams=None):
        """Element-by-element comparison of one step on every oracle stream:
        slot map, clock, counters, eviction log, miss list, slot2pos, last_use
        and LRU order always; with full_state the position->slot table and
        with contents the slot bytes, on `full_streams` (default: all of
        them).  The metadata buffer is read once."""
        cfg = self.cfg
        out = self.out_dev.cpu().numpy()
        snap = self.gpu.meta_snapshot()
        for (b, l), r in res.items():
            where = f"step {s} stream (b={b}, l={l})"
            assert r.status == 0, where
            deep = full_streams is None or (b, l) in full_streams
            np.testing.assert_array_equal(out[l, b], r.out, err_msg=f"out_slot {where}")
            g = self.gpu.state(b, l, with_pos2slot=full_state and deep, snap=snap)
            hdr = g["hdr"]
            c = r.counters
            assert hdr[hb.HDR_T] == self.oracle.st[(b, l)].t[0], f"clock {where}"
            assert hdr[hb.HDR_STATUS] == 0, where
            got = [int(hdr[i]) for i in (hb.HDR_PAD, hb.HDR_RES, hb.HDR_HIT, hb.HDR_MISS,
                                         hb.HDR_EVICT, hb.HDR_BYTES)]
            want = [c["n_pad"], c["n_res"], c["n_hit"], c["n_miss"], c["n_evict"], c["bytes"]]
            assert got == want, f"counters {where}: {got} != {want}"
            m = c["n_miss"]
            np.testing.assert_array_equal(g["evict"][:m, 0], r.log_slot, err_msg=f"evict slots {where}")
            np.testing.assert_array_equal(g["evict"][:m, 1], r.log_old, err_msg=f"evict old {where}")
            np.testing.assert_array_equal(g["miss"][:m, 0], r.log_slot, err_msg=f"miss slots {where}")
            ost = self.oracle.st[(b, l)]
            np.testing.assert_array_equal(g["miss"][:m, 1], ost.slot2pos[r.log_slot],
                                          err_msg=f"miss positions {where}")
            np.testing.assert_array_equal(g["slot2pos"], ost.slot2pos, err_msg=f"slot2pos {where}")
            np.testing.assert_array_equal(g["last_use"], ost.last_use, err_msg=f"last_use {where}")
            # the maintained LRU order is the (last_use, slot) sort of the slots
            want_order = np.lexsort((np.arange(cfg.C), ost.last_use))
            np.testing.assert_array_equal(g["order"], want_order, err_msg=f"lru order {where}")
            if full_state and deep:
                np.testing.assert_array_equal(g["pos2slot"], ost.pos2slot,
                                              err_msg=f"pos2slot {where}")
            if contents and deep and not self.no_io:
                self.compare_contents(b, l, s, host_rows=host_rows)

    def compare_contents(self, b, l, s, host_rows=True):
        """Every filled LRU slot and every current window slot holds the same
        bytes as the oracle's slot and (unless the caller has changed host
        rows since they were fetched) as the host row it stands for."""
        cfg = self.cfg
        ost = self.oracle.st[(b, l)]
        dev = self.gpu.slots(b, l)
        filled = np.nonzero(ost.slot2pos >= 0)[0]
        where = f"step {s} stream (b={b}, l={l})"
        np.testing.assert_array_equal(dev[filled], ost.slots[filled], err_msg=f"slot bytes {where}")
        host = self.gpu.host(b, l)
        if host_rows:
            np.testing.assert_array_equal(dev[filled], host[ost.slot2pos[filled]],
                                          err_msg=f"slot vs host row {where}")
        if cfg.R:
            ctx = cfg.ctx_at(s)
            win = np.arange(max(0, ctx - cfg.R), ctx)
            ring = cfg.C + win % cfg.R
            if host_rows:
                np.testing.assert_array_equal(dev[ring], host[win], err_msg=f"window bytes {where}")
            np.testing.assert_array_equal(dev[ring], ost.slots[ring], err_msg=f"window vs oracle {where}")

    def close(self):
        self.gpu.close()
