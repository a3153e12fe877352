"""Thin wrappers with the C names: torch tensors in, raw pointers to the C ABI.

Every function checks the status the library returns and raises HsError on
anything but HS_OK.  Streams default to torch's current stream, so the calls
order with surrounding torch work exactly as the C calls would.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import HS_OK, HsBatch, HsError, HsLayout, lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("tensors passed to the library must be contiguous")
        return t.data_ptr()
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, what: str) -> None:
    if status != HS_OK:
        detail = lib().hs_last_error().decode() if status in (3, 4) else ""
        raise HsError(status, f"{what} failed ({hs_status_string(status)}"
                              f"{'; ' + detail if detail else ''})")


def hs_status_string(status: int) -> str:
    return lib().hs_status_string(status).decode()


def layout_of(page_size: int, row_bytes: int, num_layers: int, hot_capacity: int,
              pool_rows: int, host_rows: int, pool_layer_stride: int | None = None,
              host_layer_stride: int | None = None) -> HsLayout:
    return HsLayout(page_size, row_bytes, num_layers, hot_capacity, pool_rows, host_rows,
                    pool_layer_stride if pool_layer_stride is not None else pool_rows * row_bytes,
                    host_layer_stride if host_layer_stride is not None else host_rows * row_bytes)


def batch_of(num_reqs: int, max_pages: int, kv_pool, host_pool, block_table, host_block_table,
             ctx_len, hot_blocks, slot_token, slot_stamp, fill_sync=None,
             fill_sync_words: int | None = None) -> HsBatch:
    """kv_pool and the tables are CUDA tensors; host_pool is a HostPool, a
    device-visible address (int), or None when host_rows is 0; fill_sync is
    None or zeroed int32 device words (at least HS_FILL_SYNC_WORDS): a CUDA
    tensor, whose length is the word count unless fill_sync_words says
    otherwise, or an address with fill_sync_words."""
    hp = host_pool.device_ptr if isinstance(host_pool, HostPool) else _ptr(host_pool)
    if isinstance(fill_sync, torch.Tensor) and fill_sync.dtype != torch.int32:
        raise TypeError(f"fill_sync must be int32, not {fill_sync.dtype}")
    if fill_sync_words is None:
        fill_sync_words = fill_sync.numel() if isinstance(fill_sync, torch.Tensor) else 0
    return HsBatch(num_reqs, max_pages, _ptr(kv_pool), hp, _ptr(block_table),
                   _ptr(host_block_table), _ptr(ctx_len), _ptr(hot_blocks), _ptr(slot_token),
                   _ptr(slot_stamp), _ptr(fill_sync), fill_sync_words)


def hs_resolve(layout: HsLayout, batch: HsBatch, topk, top_k: int, stamp: int, row_ids,
               gather_out, stats, stream=None) -> None:
    _check(lib().hs_resolve(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk), top_k,
                            ctypes.c_uint32(stamp), _ptr(row_ids), _ptr(gather_out), _ptr(stats),
                            _stream(stream)), "hs_resolve")


def hs_plan_replay(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int, stamp: int,
                   row_ids, gather_out, stats, offload_pairs=None, n_offload: int = 0,
                   stream=None) -> None:
    _check(lib().hs_plan_replay(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk), num_pos,
                                top_k, ctypes.c_uint32(stamp), _ptr(row_ids), _ptr(gather_out),
                                _ptr(stats), _ptr(offload_pairs), n_offload, _stream(stream)),
           "hs_plan_replay")


def hs_resolve_grouped(layout: HsLayout, batch: HsBatch, group_layers: int, topk, num_pos: int,
                       top_k: int, stamp: int, row_ids, gather_out, stats, offload_pairs=None,
                       n_offload: int = 0, stream=None) -> None:
    _check(lib().hs_resolve_grouped(ctypes.byref(layout), ctypes.byref(batch), group_layers,
                                    _ptr(topk), num_pos, top_k, ctypes.c_uint32(stamp),
                                    _ptr(row_ids), _ptr(gather_out), _ptr(stats),
                                    _ptr(offload_pairs), n_offload, _stream(stream)),
           "hs_resolve_grouped")


def hs_resolve_decide(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int,
                      stamp: int, row_ids, gather_out, stats, stream=None) -> None:
    _check(lib().hs_resolve_decide(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk), num_pos,
                                   top_k, ctypes.c_uint32(stamp), _ptr(row_ids), _ptr(gather_out),
                                   _ptr(stats), _stream(stream)), "hs_resolve_decide")


def hs_resolve_fetch(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int,
                     gather_out, stream=None) -> None:
    _check(lib().hs_resolve_fetch(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk), num_pos,
                                  top_k, _ptr(gather_out), _stream(stream)), "hs_resolve_fetch")


def hs_resolve_move(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int, row_ids,
                    gather_out, stream=None) -> None:
    _check(lib().hs_resolve_move(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk), num_pos,
                                 top_k, _ptr(row_ids), _ptr(gather_out), _stream(stream)),
           "hs_resolve_move")


def hs_resolve_commit(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int, row_ids,
                      gather_out, stream=None) -> None:
    _check(lib().hs_resolve_commit(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk),
                                   num_pos, top_k, _ptr(row_ids), _ptr(gather_out),
                                   _stream(stream)), "hs_resolve_commit")


def hs_gather(layout: HsLayout, kv_pool, row_ids, num_reqs: int, rows_per_req_layer: int, out,
              stream=None) -> None:
    _check(lib().hs_gather(ctypes.byref(layout), _ptr(kv_pool), _ptr(row_ids), num_reqs,
                           rows_per_req_layer, _ptr(out), _stream(stream)), "hs_gather")


def hs_offload_prefix_pages(layout: HsLayout, kv_pool, host_pool, pairs, n: int,
                            stream=None) -> None:
    hp = host_pool.device_ptr if isinstance(host_pool, HostPool) else _ptr(host_pool)
    _check(lib().hs_offload_prefix_pages(ctypes.byref(layout), _ptr(kv_pool), hp, _ptr(pairs), n,
                                         _stream(stream)), "hs_offload_prefix_pages")


def hs_page_touch(layout: HsLayout, batch: HsBatch, topk, entries_per_req: int, stamp: int,
                  page_use, stream=None) -> None:
    _check(lib().hs_page_touch(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk),
                               entries_per_req, stamp, _ptr(page_use), _stream(stream)),
           "hs_page_touch")


def hs_resolve_in_place(layout: HsLayout, batch: HsBatch, topk, num_pos: int, top_k: int,
                        stamp: int, row_ids, staging, stats, offload_pairs=None, n_offload: int = 0,
                        stream=None) -> None:
    _check(lib().hs_resolve_in_place(ctypes.byref(layout), ctypes.byref(batch), _ptr(topk),
                                     num_pos, top_k, ctypes.c_uint32(stamp), _ptr(row_ids),
                                     _ptr(staging), _ptr(stats), _ptr(offload_pairs), n_offload,
                                     _stream(stream)), "hs_resolve_in_place")


def hs_sparse_mla_workspace_bytes(num_tokens: int, num_heads: int, top_k: int) -> int:
    return int(lib().hs_sparse_mla_workspace_bytes(num_tokens, num_heads, top_k))


def hs_sparse_mla_decode(layout: HsLayout, kv_layer, row_ids, num_tokens: int, top_k: int, q,
                         num_heads: int, sm_scale: float, out, lse, workspace=None,
                         workspace_bytes: int = 0, stream=None) -> None:
    """kv_layer: a uint8 device tensor (one layer of the pool) or a device
    address; workspace: a device tensor of hs_sparse_mla_workspace_bytes."""
    kv = kv_layer if isinstance(kv_layer, int) else _ptr(kv_layer)
    if workspace is not None and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().hs_sparse_mla_decode(ctypes.byref(layout), kv, _ptr(row_ids), num_tokens, top_k,
                                      _ptr(q), num_heads, sm_scale, _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace_bytes, _stream(stream)),
           "hs_sparse_mla_decode")


def hs_sparse_mla_decode_noalloc(layout: HsLayout, kv_layer, row_ids, num_tokens: int,
                                 top_k: int, q, num_heads: int, sm_scale: float, out, lse,
                                 stream=None) -> None:
    """hs_sparse_mla_decode with the library's per-device workspace."""
    kv = kv_layer if isinstance(kv_layer, int) else _ptr(kv_layer)
    _check(lib().hs_sparse_mla_decode_noalloc(ctypes.byref(layout), kv, _ptr(row_ids), num_tokens,
                                              top_k, _ptr(q), num_heads, sm_scale, _ptr(out),
                                              _ptr(lse), _stream(stream)),
           "hs_sparse_mla_decode_noalloc")


def hs_sparse_mla_noalloc_max_workspace() -> int:
    return int(lib().hs_sparse_mla_noalloc_max_workspace())


def hs_host_alloc(nbytes: int) -> int:
    p = ctypes.c_void_p()
    _check(lib().hs_host_alloc(nbytes, ctypes.byref(p)), "hs_host_alloc")
    return p.value


def hs_host_free(ptr: int) -> None:
    _check(lib().hs_host_free(ptr), "hs_host_free")


def hs_host_device_pointer(ptr: int) -> int:
    d = ctypes.c_void_p()
    _check(lib().hs_host_device_pointer(ptr, ctypes.byref(d)), "hs_host_device_pointer")
    return d.value


class HostPool:
    """Pinned, device-mapped host memory holding the host pool.

    ``array`` is a numpy uint8 view of the whole allocation (host side);
    ``tensor`` the same memory as a CPU torch tensor; ``device_ptr`` the
    address kernels read and write.
    """

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.host_ptr = hs_host_alloc(self.nbytes)
        self.device_ptr = hs_host_device_pointer(self.host_ptr)
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.host_ptr)
        self.array = np.frombuffer(buf, dtype=np.uint8)
        self.tensor = torch.from_numpy(self.array)

    def close(self) -> None:
        if self.host_ptr:
            self.tensor = None
            self.array = None
            hs_host_free(self.host_ptr)
            self.host_ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
