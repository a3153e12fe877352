"""Loading ``libhisparse.so`` and the ctypes mirror of ``include/hisparse.h``."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhisparse.so")

HS_OK = 0
HS_ERR_INVALID_ARGUMENT = 1
HS_ERR_UNSUPPORTED = 2
HS_ERR_LAUNCH = 3
HS_ERR_HIP = 4
HS_MAX_ENTRIES = 8192
HS_MAX_HOT_CAPACITY = 12288
HS_MAX_ROW_BYTES = 4096
HS_FILL_SYNC_WORDS = 64

EXPORTS = ("hs_resolve", "hs_gather", "hs_offload_prefix_pages", "hs_plan_replay",
           "hs_resolve_grouped",
           "hs_resolve_decide", "hs_resolve_fetch", "hs_resolve_move", "hs_resolve_commit",
           "hs_page_touch", "hs_resolve_in_place", "hs_sparse_mla_decode", "hs_sparse_mla_workspace_bytes",
           "hs_sparse_mla_decode_noalloc", "hs_sparse_mla_noalloc_max_workspace",
           "hs_status_string", "hs_last_error", "hs_host_alloc", "hs_host_free",
           "hs_host_device_pointer")


class HsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status}")


class HsLayout(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("row_bytes", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("hot_capacity", ctypes.c_int32),
                ("pool_rows", ctypes.c_int64), ("host_rows", ctypes.c_int64),
                ("pool_layer_stride", ctypes.c_int64), ("host_layer_stride", ctypes.c_int64)]


class HsBatch(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("kv_pool", ctypes.c_void_p), ("host_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("host_block_table", ctypes.c_void_p),
                ("ctx_len", ctypes.c_void_p), ("hot_blocks", ctypes.c_void_p),
                ("slot_token", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("fill_sync", ctypes.c_void_p), ("fill_sync_words", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built or fails to load:
    there is deliberately no fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        lay, bat = ctypes.POINTER(HsLayout), ctypes.POINTER(HsBatch)
        L.hs_resolve.argtypes = [lay, bat, vp, i32, u32, vp, vp, vp, vp]
        L.hs_gather.argtypes = [lay, vp, vp, i32, i32, vp, vp]
        L.hs_offload_prefix_pages.argtypes = [lay, vp, vp, vp, i32, vp]
        L.hs_plan_replay.argtypes = [lay, bat, vp, i32, i32, u32, vp, vp, vp, vp, i32, vp]
        L.hs_resolve_grouped.argtypes = [lay, bat, i32, vp, i32, i32, u32, vp, vp, vp, vp, i32, vp]
        L.hs_resolve_decide.argtypes = [lay, bat, vp, i32, i32, u32, vp, vp, vp, vp]
        L.hs_resolve_fetch.argtypes = [lay, bat, vp, i32, i32, vp, vp]
        L.hs_resolve_move.argtypes = [lay, bat, vp, i32, i32, vp, vp, vp]
        L.hs_resolve_commit.argtypes = [lay, bat, vp, i32, i32, vp, vp, vp]
        L.hs_page_touch.argtypes = [lay, bat, vp, i32, u32, vp, vp]
        L.hs_resolve_in_place.argtypes = [lay, bat, vp, i32, i32, u32, vp, vp, vp, vp, i32, vp]
        L.hs_sparse_mla_decode.argtypes = [lay, vp, vp, i32, i32, vp, i32, ctypes.c_float, vp,
                                           vp, vp, sz, vp]
        L.hs_sparse_mla_workspace_bytes.argtypes = [i32, i32, i32]
        L.hs_sparse_mla_decode_noalloc.argtypes = [lay, vp, vp, i32, i32, vp, i32,
                                                   ctypes.c_float, vp, vp, vp]
        L.hs_sparse_mla_noalloc_max_workspace.argtypes = []
        L.hs_status_string.argtypes = [i32]
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_last_error.argtypes = []
        L.hs_last_error.restype = ctypes.c_char_p
        L.hs_host_alloc.argtypes = [sz, ctypes.POINTER(vp)]
        L.hs_host_free.argtypes = [vp]
        L.hs_host_device_pointer.argtypes = [vp, ctypes.POINTER(vp)]
        for name in EXPORTS:
            if name in ("hs_status_string", "hs_last_error"):
                continue
            getattr(L, name).restype = i32
        L.hs_sparse_mla_workspace_bytes.restype = sz
        L.hs_sparse_mla_noalloc_max_workspace.restype = sz
        _lib = L
    return _lib
