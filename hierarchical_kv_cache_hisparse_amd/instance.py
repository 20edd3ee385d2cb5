"""Device-side owner of one libhisparse instance: pinned host histories
(hisparse_host_alloc on the GPU's NUMA node), the caller-owned cache and
metadata buffers (torch device memory), the handle, and read-back views of
the per-stream state.  Allocation and argument marshalling only: every step
of the method runs in the library's kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import binding as hb


def host_view(ptr: int, nbytes: int) -> np.ndarray:
    return np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(ptr))


class GpuInstance:
    """A libhisparse handle over pinned host histories and torch device memory.

    cfg: a workload shape (B, layers, l_cap, row_bytes, C, R, k); hosts: an
    existing {(b, l): (ptr, view)} map to share another instance's histories.
    """

    def __init__(self, cfg, flags: int = 0, host_flags: int = hb.HISPARSE_HOST_COHERENT,
                 device: str = "cuda:0", hosts=None, numa_node: int = hb.HISPARSE_NUMA_DEVICE):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = device
        self.flags = flags
        self.hcfg = hb.make_config(cfg.B, cfg.layers, cfg.l_cap, cfg.row_bytes, cfg.C, cfg.R,
                                   cfg.k, flags)
        cache_bytes, meta_bytes = hb.hisparse_workspace_bytes(self.hcfg)
        self.lay = hb.hisparse_meta_layout_of(self.hcfg)
        nbytes = cfg.l_cap * cfg.row_bytes
        self.owns_hosts = hosts is None
        if hosts is None:
            hosts = {}
            for l in range(cfg.layers):
                for b in range(cfg.B):
                    ptr = hb.hisparse_host_alloc(nbytes, host_flags, numa_node)
                    hosts[(b, l)] = (ptr, host_view(ptr, nbytes).reshape(cfg.l_cap, cfg.row_bytes))
        self.hosts = hosts
        self.cache = torch.empty(cache_bytes, dtype=torch.uint8, device=device)
        self.meta = torch.empty(meta_bytes, dtype=torch.uint8, device=device)
        ptrs = [hosts[(b, l)][0] for l in range(cfg.layers) for b in range(cfg.B)]
        self.h = hb.hisparse_create(self.hcfg, ptrs, self.cache.data_ptr(), self.meta.data_ptr())

    def host(self, b: int, l: int) -> np.ndarray:
        return self.hosts[(b, l)][1]

    @property
    def stream(self) -> int:
        return self.torch.cuda.current_stream().cuda_stream

    def close(self):
        if self.h is not None:
            hb.hisparse_destroy(self.h)
            self.h = None
        if self.owns_hosts:
            for ptr, _ in self.hosts.values():
                hb.hisparse_host_free(ptr)
            self.hosts = {}

    # -- state read-back ------------------------------------------------------
    def _block(self, b: int, l: int):
        return self.lay.stream_base + (l * self.cfg.B + b) * self.lay.stream_stride

    def _i32(self, b, l, off, n, snap=None):
        start = self._block(b, l) + off
        if snap is not None:   # a host copy of the whole buffer (meta_snapshot)
            return snap[start: start + 4 * n].view(np.int32)
        return self.meta[start: start + 4 * n].view(self.torch.int32).cpu().numpy()

    def meta_snapshot(self) -> np.ndarray:
        """The whole metadata buffer copied to the host in one transfer, for
        reading many streams' state (pass it to hdr / state as ``snap``)."""
        return self.meta.cpu().numpy()

    def hdr(self, b, l, snap=None):
        return self._i32(b, l, self.lay.hdr, 16, snap)

    def state(self, b, l, with_pos2slot=True, snap=None):
        c = self.cfg
        st = {"hdr": self.hdr(b, l, snap),
              "slot2pos": self._i32(b, l, self.lay.slot2pos, c.C, snap),
              "last_use": self._i32(b, l, self.lay.last_use, c.C, snap),
              "order": self._i32(b, l, self.lay.lru_order, c.C, snap),
              "evict": self._i32(b, l, self.lay.evict_log, 2 * c.k, snap).reshape(c.k, 2),
              "miss": self._i32(b, l, self.lay.miss_list, 2 * c.k, snap).reshape(c.k, 2)}
        if with_pos2slot:
            st["pos2slot"] = self._i32(b, l, self.lay.pos2slot, c.l_cap, snap)
        return st

    def totals(self, snap=None) -> np.ndarray:
        """int64 [3]: running misses, evictions and hits summed over every stream."""
        snap = self.meta_snapshot() if snap is None else snap
        tot = np.zeros(3, np.int64)
        for l in range(self.cfg.layers):
            for b in range(self.cfg.B):
                h = self.hdr(b, l, snap)
                for i, w in enumerate((hb.HDR_TOTAL_MISS, hb.HDR_TOTAL_EVICT, hb.HDR_TOTAL_HIT)):
                    tot[i] += int(h[w:w + 2].view(np.int64)[0])
        return tot

    def slots(self, b, l) -> np.ndarray:
        c = self.cfg
        per = (c.C + c.R) * c.row_bytes
        start = (l * c.B + b) * per
        return self.cache[start: start + per].cpu().numpy().reshape(c.C + c.R, c.row_bytes)

    def status(self, clear=False) -> int:
        return hb.hisparse_get_status(self.h, clear)
