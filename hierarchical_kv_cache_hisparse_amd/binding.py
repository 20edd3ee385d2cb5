"""Thin ctypes binding of libhisparse (include/hisparse.h).

Argument marshalling only: every function has the C name, takes plain
integers for device/host pointers and HIP stream handles (e.g.
``tensor.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``), and
raises ``HisparseError`` on a negative return code.  All computation happens
in the library's HIP kernels; there is no fallback of any kind, and importing
this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhisparse.so")

HISPARSE_OK = 0
HISPARSE_ERR_INVALID_ARG = -1
HISPARSE_ERR_OOM = -2
HISPARSE_ERR_HIP = -3
HISPARSE_ERR_STATE = -4
HISPARSE_ERR_UNSUPPORTED = -5

HISPARSE_NO_IO = 0x1
HISPARSE_DEBUG_VALIDATE = 0x2
HISPARSE_SERIALIZE_PREFETCH = 0x4

HISPARSE_STATUS_SEL_RANGE = 0x1
HISPARSE_STATUS_SEL_DUP = 0x2
HISPARSE_STATUS_CTX_RANGE = 0x4
HISPARSE_STATUS_PREFETCH_MISMATCH = 0x8

HISPARSE_HOST_COHERENT = 0x0
HISPARSE_HOST_NONCOHERENT = 0x1

HISPARSE_NUMA_DEVICE = -1      # the NUMA node closest to the current device
HISPARSE_NUMA_DEFAULT = -2     # the process's own memory policy

# Per-stream header words (int32) in the metadata buffer.
HDR_T, HDR_STATUS, HDR_PAD, HDR_RES, HDR_HIT, HDR_MISS, HDR_EVICT, HDR_BYTES = range(8)
HDR_TOTAL_MISS, HDR_TOTAL_EVICT, HDR_TOTAL_HIT = 8, 10, 12   # int64 word pairs


class hisparse_config(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("max_positions", ctypes.c_int64),
        ("row_bytes", ctypes.c_int32),
        ("cache_slots", ctypes.c_int32),
        ("resident_window", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class hisparse_meta_layout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t) for name in (
        "total_bytes", "status", "stream_base", "stream_stride", "hdr", "pos2slot",
        "slot2pos", "last_use", "lru_order", "evict_log", "miss_list")]


class hisparse_timing(ctypes.Structure):
    _fields_ = [
        ("resolve_launches", ctypes.c_int64),
        ("fetch_launches", ctypes.c_int64),
        ("resolve_ms", ctypes.c_double),
        ("fetch_ms", ctypes.c_double),
    ]


class HisparseError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where} failed: {detail} (code {code})")
        self.code = code


_lib = None


def library():
    """The loaded libhisparse.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with `python -m "
                "hierarchical_kv_cache_hisparse_amd.build` (or __graft_entry__.build())")
        # One HIP runtime per process: PyTorch ships its own libamdhip64.so.7.
        # Loading torch first makes the library bind to that runtime by soname
        # instead of pulling in a second one (which leaves torch without a GPU).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        sig = {
            "hisparse_workspace_bytes": [P, P, P],
            "hisparse_meta_layout_of": [P, P],
            "hisparse_host_alloc": [SZ, ctypes.c_int, U32, P],
            "hisparse_host_numa_node": [P, P],
            "hisparse_device_numa_node": [P],
            "hisparse_host_free": [P],
            "hisparse_create": [P, P, P, P, P],
            "hisparse_destroy": [P],
            "hisparse_resolve": [P, P, P, P, I32, P],
            "hisparse_resolve_multi": [P, P, P, I32, I32, P, I32, P],
            "hisparse_prefetch": [P, P, P, P, P, I32, P],
            "hisparse_load_window": [P, P, I32, P],
            "hisparse_append": [P, P, I32, P, P],
            "hisparse_append_resolve": [P, P, I32, P, P, P, P, P],
            "hisparse_append_resolve_multi": [P, P, I32, P, P, P, I32, I32, P, P],
            "hisparse_reset": [P, P, I32, I32],
            "hisparse_get_status": [P, P, ctypes.c_int],
            "hisparse_set_timing": [P, ctypes.c_int],
            "hisparse_get_timing": [P, P],
            "hisparse_probe_host_read": [P, P, P, SZ, I32],
            "hisparse_mla_workspace_bytes": [P, I32, P],
            "hisparse_sparse_mla_decode": [P, P, I32, P, P, I32, ctypes.c_float, P, P, P],
            "hisparse_mla_workspace_bytes_multi": [P, I32, I32, I32, P],
            "hisparse_sparse_mla_decode_multi": [P, P, I32, I32, I32, P, P, I32, ctypes.c_float, P,
                                                 P, P],
            "hisparse_sparse_mla_decode_noalloc": [P, P, I32, P, P, I32, ctypes.c_float, P, P],
            "hisparse_topk_workspace_bytes": [I32, ctypes.c_int64, P],
            "hisparse_topk": [P, P, ctypes.c_int64, I32, ctypes.c_int64, P, I32, P, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.hisparse_strerror.argtypes = [ctypes.c_int]
        lib.hisparse_strerror.restype = ctypes.c_char_p
        lib.hisparse_last_error.argtypes = []
        lib.hisparse_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != HISPARSE_OK:
        lib = library()
        detail = lib.hisparse_last_error().decode(errors="replace") or \
            lib.hisparse_strerror(rc).decode()
        raise HisparseError(rc, where, detail)


def make_config(num_requests, num_layers, max_positions, row_bytes, cache_slots,
                resident_window, top_k, flags=0) -> hisparse_config:
    return hisparse_config(num_requests, num_layers, max_positions, row_bytes, cache_slots,
                           resident_window, top_k, flags)


def hisparse_workspace_bytes(cfg: hisparse_config) -> tuple[int, int]:
    cache, meta = ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().hisparse_workspace_bytes(ctypes.byref(cfg), ctypes.byref(cache),
                                              ctypes.byref(meta)), "hisparse_workspace_bytes")
    return cache.value, meta.value


def hisparse_meta_layout_of(cfg: hisparse_config) -> hisparse_meta_layout:
    out = hisparse_meta_layout()
    _check(library().hisparse_meta_layout_of(ctypes.byref(cfg), ctypes.byref(out)),
           "hisparse_meta_layout_of")
    return out


def hisparse_host_alloc(nbytes: int, flags: int = HISPARSE_HOST_COHERENT,
                        numa_node: int = HISPARSE_NUMA_DEVICE) -> int:
    ptr = ctypes.c_void_p()
    _check(library().hisparse_host_alloc(nbytes, numa_node, flags, ctypes.byref(ptr)),
           "hisparse_host_alloc")
    return ptr.value


def hisparse_host_numa_node(host_ptr: int) -> int:
    node = ctypes.c_int()
    _check(library().hisparse_host_numa_node(host_ptr, ctypes.byref(node)),
           "hisparse_host_numa_node")
    return node.value


def hisparse_device_numa_node() -> int:
    node = ctypes.c_int()
    _check(library().hisparse_device_numa_node(ctypes.byref(node)), "hisparse_device_numa_node")
    return node.value


def hisparse_host_free(ptr: int) -> None:
    _check(library().hisparse_host_free(ptr), "hisparse_host_free")


def hisparse_create(cfg: hisparse_config, host_rows, device_cache: int, device_meta: int):
    arr = (ctypes.c_void_p * len(host_rows))(*host_rows)
    h = ctypes.c_void_p()
    _check(library().hisparse_create(ctypes.byref(cfg), arr, device_cache, device_meta,
                                     ctypes.byref(h)), "hisparse_create")
    return h


def hisparse_destroy(h) -> None:
    _check(library().hisparse_destroy(h), "hisparse_destroy")


def hisparse_resolve(h, stream: int, sel: int, ctx_len: int, layer: int, out_slot: int) -> None:
    _check(library().hisparse_resolve(h, stream, sel, ctx_len, layer, out_slot),
           "hisparse_resolve")


def hisparse_resolve_multi(h, stream: int, sel: int, queries: int, per_query: int, ctx_len: int,
                           layer: int, out_slot: int) -> None:
    _check(library().hisparse_resolve_multi(h, stream, sel, queries, per_query, ctx_len, layer,
                                            out_slot), "hisparse_resolve_multi")


def hisparse_prefetch(h, main_stream: int, side_stream: int, sel: int, ctx_len: int,
                      layer: int, out_slot: int = 0) -> None:
    _check(library().hisparse_prefetch(h, main_stream, side_stream, sel, ctx_len, layer,
                                       out_slot or None),
           "hisparse_prefetch")


def hisparse_load_window(h, stream: int, layer: int, ctx_len: int) -> None:
    _check(library().hisparse_load_window(h, stream, layer, ctx_len), "hisparse_load_window")


def hisparse_append(h, stream: int, layer: int, rows: int, pos: int) -> None:
    _check(library().hisparse_append(h, stream, layer, rows, pos), "hisparse_append")


def hisparse_append_resolve(h, stream: int, layer: int, rows: int, pos: int, sel: int,
                            ctx_len: int, out_slot: int) -> None:
    _check(library().hisparse_append_resolve(h, stream, layer, rows, pos, sel, ctx_len, out_slot),
           "hisparse_append_resolve")


def hisparse_append_resolve_multi(h, stream: int, layer: int, rows: int, pos: int, sel: int,
                                  queries: int, per_query: int, ctx_len: int,
                                  out_slot: int) -> None:
    _check(library().hisparse_append_resolve_multi(h, stream, layer, rows, pos, sel, queries,
                                                   per_query, ctx_len, out_slot),
           "hisparse_append_resolve_multi")


def hisparse_reset(h, stream: int, layer: int = -1, request: int = -1) -> None:
    _check(library().hisparse_reset(h, stream, layer, request), "hisparse_reset")


def hisparse_get_status(h, clear: bool = False) -> int:
    st = ctypes.c_uint32()
    _check(library().hisparse_get_status(h, ctypes.byref(st), 1 if clear else 0),
           "hisparse_get_status")
    return st.value


def hisparse_set_timing(h, enable: bool) -> None:
    _check(library().hisparse_set_timing(h, 1 if enable else 0), "hisparse_set_timing")


def hisparse_get_timing(h) -> dict:
    t = hisparse_timing()
    _check(library().hisparse_get_timing(h, ctypes.byref(t)), "hisparse_get_timing")
    return {"resolve_launches": t.resolve_launches, "fetch_launches": t.fetch_launches,
            "resolve_ms": t.resolve_ms, "fetch_ms": t.fetch_ms}


def hisparse_probe_host_read(stream: int, host: int, device: int, nbytes: int,
                             workgroups: int) -> None:
    _check(library().hisparse_probe_host_read(stream, host, device, nbytes, workgroups),
           "hisparse_probe_host_read")


def hisparse_strerror(code: int) -> str:
    return library().hisparse_strerror(code).decode()


def hisparse_last_error() -> str:
    return library().hisparse_last_error().decode(errors="replace")


def hisparse_mla_workspace_bytes(h, num_heads: int) -> int:
    n = ctypes.c_size_t()
    _check(library().hisparse_mla_workspace_bytes(h, num_heads, ctypes.byref(n)),
           "hisparse_mla_workspace_bytes")
    return n.value


def hisparse_sparse_mla_decode(h, stream: int, layer: int, q: int, out_slot: int,
                               num_heads: int, scale: float, workspace: int, out: int,
                               lse: int) -> None:
    _check(library().hisparse_sparse_mla_decode(h, stream, layer, q, out_slot, num_heads,
                                                scale, workspace, out, lse),
           "hisparse_sparse_mla_decode")


HISPARSE_NOALLOC_SCRATCH_BYTES = 40 << 20


def hisparse_sparse_mla_decode_noalloc(h, stream: int, layer: int, q: int, out_slot: int,
                                       num_heads: int, scale: float, out: int, lse: int) -> None:
    _check(library().hisparse_sparse_mla_decode_noalloc(h, stream, layer, q, out_slot, num_heads,
                                                        scale, out, lse),
           "hisparse_sparse_mla_decode_noalloc")


def hisparse_mla_workspace_bytes_multi(h, queries: int, per_query: int, num_heads: int) -> int:
    n = ctypes.c_size_t()
    _check(library().hisparse_mla_workspace_bytes_multi(h, queries, per_query, num_heads,
                                                        ctypes.byref(n)),
           "hisparse_mla_workspace_bytes_multi")
    return n.value


def hisparse_sparse_mla_decode_multi(h, stream: int, layer: int, queries: int, per_query: int,
                                     q: int, out_slot: int, num_heads: int, scale: float,
                                     workspace: int, out: int, lse: int) -> None:
    _check(library().hisparse_sparse_mla_decode_multi(h, stream, layer, queries, per_query, q,
                                                      out_slot, num_heads, scale, workspace, out,
                                                      lse),
           "hisparse_sparse_mla_decode_multi")


def hisparse_topk_workspace_bytes(num_rows: int, max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(library().hisparse_topk_workspace_bytes(num_rows, max_len, ctypes.byref(n)),
           "hisparse_topk_workspace_bytes")
    return n.value


def hisparse_topk(stream: int, scores: int, row_stride: int, num_rows: int, max_len: int,
                  ctx_len: int, k: int, workspace: int, out_sel: int) -> None:
    _check(library().hisparse_topk(stream, scores, row_stride, num_rows, max_len, ctx_len, k,
                                   workspace, out_sel), "hisparse_topk")
