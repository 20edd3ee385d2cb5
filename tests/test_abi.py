"""The C-ABI library loads and exports every symbol include/hisparse.h
declares, and its host-only logic (shape validation, workspace sizes, the
metadata layout, error strings) behaves as documented (no GPU needed)."""
import ctypes
import os
import re

import pytest

from hierarchical_kv_cache_hisparse_amd import binding as hb
from workload import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hisparse_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("hisparse_create", "hisparse_resolve", "hisparse_prefetch", "hisparse_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hb.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_has_the_same_names():
    missing = [n for n in declared_functions() if not hasattr(hb, n)]
    assert not missing, missing


def _cfg(w, flags=0):
    return hb.make_config(w.B, w.layers, w.l_cap, w.row_bytes, w.C, w.R, w.k, flags)


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workspace_sizes_of_the_workloads(cfg_id):
    w = WORKLOADS[cfg_id]
    cache, meta = hb.hisparse_workspace_bytes(_cfg(w))
    assert cache == w.layers * w.B * (w.C + w.R) * w.row_bytes
    lay = hb.hisparse_meta_layout_of(_cfg(w))
    assert lay.total_bytes == meta
    offs = [lay.hdr, lay.pos2slot, lay.slot2pos, lay.last_use, lay.lru_order, lay.evict_log,
            lay.miss_list]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.slot2pos - lay.pos2slot >= 4 * w.l_cap
    assert lay.stream_stride - lay.miss_list >= 8 * w.k
    assert lay.stream_base >= 4 and lay.stream_base % 256 == 0
    assert meta == lay.stream_base + w.layers * w.B * lay.stream_stride


@pytest.mark.parametrize("field,value,code", [
    ("num_requests", 0, hb.HISPARSE_ERR_INVALID_ARG),
    ("num_layers", 0, hb.HISPARSE_ERR_INVALID_ARG),
    ("max_positions", 0, hb.HISPARSE_ERR_INVALID_ARG),
    ("max_positions", 1 << 31, hb.HISPARSE_ERR_INVALID_ARG),
    ("row_bytes", 1000, hb.HISPARSE_ERR_INVALID_ARG),
    ("row_bytes", 0, hb.HISPARSE_ERR_INVALID_ARG),
    ("cache_slots", 100, hb.HISPARSE_ERR_INVALID_ARG),      # C < k
    ("resident_window", -1, hb.HISPARSE_ERR_INVALID_ARG),
    ("top_k", 0, hb.HISPARSE_ERR_INVALID_ARG),
    ("top_k", 8192, hb.HISPARSE_ERR_INVALID_ARG),          # > C
    ("flags", 0x100, hb.HISPARSE_ERR_INVALID_ARG),
    ("cache_slots", 20000, hb.HISPARSE_ERR_UNSUPPORTED),
])
def test_invalid_configs_are_rejected_on_the_host(field, value, code):
    cfg = _cfg(WORKLOADS[2])
    setattr(cfg, field, value)
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_workspace_bytes(cfg)
    assert e.value.code == code
    assert hb.hisparse_last_error()


def test_largest_shape_fits_the_lds():
    """C = 16384 and k = 4096 with the debug hash is the largest shape; its
    resolve workgroup still fits gfx950's 160 KiB of LDS."""
    cfg = hb.make_config(1, 1, 1 << 20, 1152, 16384, 0, 4096, hb.HISPARSE_DEBUG_VALIDATE)
    hb.hisparse_workspace_bytes(cfg)
    cfg.cache_slots = 16385
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_workspace_bytes(cfg)
    assert e.value.code == hb.HISPARSE_ERR_UNSUPPORTED


def test_error_strings():
    assert hb.hisparse_strerror(0) == "success"
    assert "invalid" in hb.hisparse_strerror(hb.HISPARSE_ERR_INVALID_ARG)
    assert hb.hisparse_strerror(-99) == "unknown error code"


def test_create_rejects_null_and_host_pointers_without_touching_them():
    cfg = _cfg(WORKLOADS[1])
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_create(cfg, [None], 0, 0)
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
    buf = (ctypes.c_uint8 * 4096)()
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_create(cfg, [ctypes.addressof(buf)], ctypes.addressof(buf),
                           ctypes.addressof(buf))
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG


def test_host_alloc_rejects_bad_arguments():
    with pytest.raises(hb.HisparseError):
        hb.hisparse_host_alloc(0)
    with pytest.raises(hb.HisparseError):
        hb.hisparse_host_alloc(4096, 0x80)
    for node in (-3, 1024):
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_host_alloc(4096, hb.HISPARSE_HOST_COHERENT, node)
        assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG


def test_host_numa_node_of_ordinary_host_memory():
    """The page-placement query is host only: on a touched buffer it names a
    node that exists on this machine, and it rejects NULL."""
    import glob
    import numpy as np
    buf = np.ones(1 << 16, np.uint8)
    node = hb.hisparse_host_numa_node(buf.ctypes.data)
    nodes = {int(p.rsplit("node", 1)[1]) for p in glob.glob("/sys/devices/system/node/node[0-9]*")}
    assert node in (nodes or {0}), (node, nodes)
    # a page the kernel cannot place-query (nothing mapped there): the only
    # node of a one-node host, else unknown
    fallback = hb.hisparse_host_numa_node(16)
    assert fallback == (next(iter(nodes)) if len(nodes) == 1 else -1), (fallback, nodes)
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_host_numa_node(None)
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG


def test_probe_and_device_node_reject_bad_arguments_before_any_launch():
    """The link probe validates its arguments on the host (no launch, no GPU
    needed): NULL buffers, an empty or non-16-byte size, no workgroups and
    buffers off 16-byte alignment are rejected; so is a NULL node pointer."""
    lib = hb.library()
    P, SZ, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    good = 4096   # never dereferenced: every call below fails its checks first
    for host, dev, nbytes, wgs in ((None, good, 1024, 4), (good, None, 1024, 4),
                                   (good, good, 0, 4), (good, good, 1000, 4),
                                   (good, good, 1024, 0), (good + 8, good, 1024, 4),
                                   (good, good + 4, 1024, 4)):
        rc = lib.hisparse_probe_host_read(P(None), P(host), P(dev), SZ(nbytes), I32(wgs))
        assert rc == hb.HISPARSE_ERR_INVALID_ARG, (host, dev, nbytes, wgs, rc)
    assert lib.hisparse_device_numa_node(None) == hb.HISPARSE_ERR_INVALID_ARG


def test_topk_workspace_sizes():
    """Per row: two 4096-bin histograms, a counter block, one bitmap word per
    32 positions rounded up to whole 4096-position chunks, and 8 bytes per
    position for boundary candidates; each part 256-byte aligned."""
    def align(x):
        return (x + 255) // 256 * 256
    for rows, n in ((1, 1), (16, 131072), (16, 262144), (4, 65536), (3, 10001)):
        words = -(-n // 4096) * 128
        want = (2 * align(rows * 4096 * 4) + align(rows * 64 * 4) + align(rows * words * 4)
                + align(rows * n * 8))
        assert hb.hisparse_topk_workspace_bytes(rows, n) == want, (rows, n)


@pytest.mark.parametrize("rows,n", [(0, 100), (65536, 100), (1, 0), (1, (1 << 31) - 4096 + 1)])
def test_topk_rejects_bad_sizes_on_the_host(rows, n):
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_topk_workspace_bytes(rows, n)
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
    with pytest.raises(hb.HisparseError):
        hb.hisparse_topk(0, 0, 4, rows, n, 0, 8, 0, 0)


def test_topk_rejects_null_and_bad_k_before_any_launch():
    for k in (0, 4097):
        with pytest.raises(hb.HisparseError) as e:
            hb.hisparse_topk(0, 256, 1024, 2, 1024, 256, k, 256, 256)
        assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
    with pytest.raises(hb.HisparseError):
        hb.hisparse_topk(0, 0, 1024, 2, 1024, 256, 8, 256, 256)


def test_multi_resolve_rejects_a_null_handle():
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_resolve_multi(None, 0, 256, 2, 8, 256, 0, 256)
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG


def test_append_resolve_rejects_a_null_handle_and_null_buffers():
    """Host-side checks of hisparse_append_resolve, before any launch."""
    with pytest.raises(hb.HisparseError) as e:
        hb.hisparse_append_resolve(None, 0, 0, 256, 256, 256, 256, 256)
    assert e.value.code == hb.HISPARSE_ERR_INVALID_ARG
