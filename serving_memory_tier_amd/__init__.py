"""Python binding of the MI355X Hybrid HiSparse hot-path library.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libhisparse.so`` (built from ``csrc/`` for gfx950).  PyTorch supplies device
memory and streams.  The names mirror the C ABI in ``include/hisparse.h``:
``hs_resolve``, ``hs_gather``, ``hs_offload_prefix_pages``, ``hs_plan_replay``,
``hs_resolve_grouped`` (layers sharing a top-K list),
the resolver's stages (``hs_resolve_decide``, ``hs_resolve_fetch``,
``hs_resolve_move``, ``hs_resolve_commit``), plus pinned host-pool helpers.  There is no fallback: if the library is
missing or fails to load, every call raises.
"""

from ._lib import (EXPORTS, HS_ERR_HIP, HS_ERR_INVALID_ARGUMENT, HS_ERR_LAUNCH,
                   HS_ERR_UNSUPPORTED, HS_FILL_SYNC_WORDS, HS_MAX_ENTRIES, HS_MAX_HOT_CAPACITY,
                   HS_MAX_ROW_BYTES,
                   HS_OK, LIB_PATH, HsBatch, HsError, HsLayout, lib)
from .api import (HostPool, batch_of, hs_gather, hs_host_alloc, hs_host_device_pointer,
                  hs_host_free, hs_offload_prefix_pages, hs_plan_replay, hs_resolve,
                  hs_resolve_commit, hs_resolve_decide, hs_resolve_fetch, hs_resolve_grouped,
                  hs_resolve_move, hs_page_touch, hs_resolve_in_place, hs_sparse_mla_decode,
                  hs_sparse_mla_workspace_bytes, hs_sparse_mla_decode_noalloc,
                  hs_sparse_mla_noalloc_max_workspace, hs_status_string, layout_of)

__all__ = [
    "EXPORTS", "HS_OK", "HS_ERR_INVALID_ARGUMENT", "HS_ERR_UNSUPPORTED", "HS_ERR_LAUNCH",
    "HS_ERR_HIP", "HS_MAX_ENTRIES", "HS_MAX_HOT_CAPACITY", "HS_MAX_ROW_BYTES", "HS_FILL_SYNC_WORDS", "LIB_PATH",
    "HsLayout", "HsBatch",
    "HsError", "HostPool", "lib", "layout_of", "batch_of", "hs_resolve", "hs_gather",
    "hs_offload_prefix_pages", "hs_plan_replay", "hs_resolve_grouped", "hs_resolve_decide",
    "hs_resolve_fetch",
    "hs_resolve_move", "hs_resolve_commit", "hs_page_touch",
    "hs_resolve_in_place", "hs_sparse_mla_decode", "hs_sparse_mla_workspace_bytes",
    "hs_sparse_mla_decode_noalloc", "hs_sparse_mla_noalloc_max_workspace", "hs_status_string", "hs_host_alloc",
    "hs_host_free", "hs_host_device_pointer",
]
