"""Python binding of the host-side residency policy (``include/hs_policy.h``,
``libhs_policy.so``): argument marshalling only.

The policy decides between decode steps which pages stay in the GPU block
pool, which become null placeholders backed by the host pool, which completed
pages are copied to host, and which pool blocks are leased to requests as
hot-buffer capacity.  Each call returns that step's edits for the GPU path's
block tables, host tables and hot-block leases.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhs_policy.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_POOL_EXHAUSTED = 2
ERR_HOST_EXHAUSTED = 3


class PolicyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status}")


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("page_size", "num_blocks", "num_host_blocks",
                                                "max_requests", "max_pages",
                                                "hot_blocks_per_request", "tail_pages")]


class _Edits(ctypes.Structure):
    _fields_ = [("bt_set", ctypes.c_void_p), ("n_bt", ctypes.c_int32), ("cap_bt", ctypes.c_int32),
                ("hbt_set", ctypes.c_void_p), ("n_hbt", ctypes.c_int32),
                ("cap_hbt", ctypes.c_int32),
                ("hot_set", ctypes.c_void_p), ("n_hot", ctypes.c_int32),
                ("cap_hot", ctypes.c_int32),
                ("reset", ctypes.c_void_p), ("n_reset", ctypes.c_int32),
                ("cap_reset", ctypes.c_int32),
                ("offload", ctypes.c_void_p), ("n_offload", ctypes.c_int32),
                ("cap_offload", ctypes.c_int32),
                ("evicted", ctypes.c_int32), ("leased", ctypes.c_int32),
                ("returned", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
        L.hs_policy_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
        L.hs_policy_destroy.argtypes = [vp]
        L.hs_policy_destroy.restype = None
        L.hs_policy_admit.argtypes = [vp, i32, i32, vp, i32, ctypes.POINTER(_Edits)]
        L.hs_policy_finish.argtypes = [vp, i32, ctypes.POINTER(_Edits)]
        L.hs_policy_step.argtypes = [vp, i32, vp, vp, i32, vp, i32, ctypes.POINTER(_Edits)]
        L.hs_policy_step_pages.argtypes = [vp, vp, vp, i32, vp, i32, ctypes.POINTER(_Edits)]
        L.hs_policy_tables.argtypes = [vp, i32, vp, vp, vp]
        L.hs_policy_free_blocks.argtypes = [vp]
        for f in (L.hs_policy_create, L.hs_policy_admit, L.hs_policy_finish, L.hs_policy_step,
                  L.hs_policy_step_pages, L.hs_policy_tables, L.hs_policy_free_blocks):
            f.restype = i32
        _lib = L
    return _lib


@dataclass
class Edits:
    """One call's edits.  Before the step: bt_set / hbt_set / hot_set rows
    (request, index, value) and the requests whose hot-buffer state must be
    cleared (``reset``).  After the step: ``offload`` (device block, host
    block) pairs."""
    bt_set: np.ndarray
    hbt_set: np.ndarray
    hot_set: np.ndarray
    reset: np.ndarray
    offload: np.ndarray
    evicted: int
    leased: int
    returned: int


class Policy:
    def __init__(self, page_size: int, num_blocks: int, num_host_blocks: int, max_requests: int,
                 max_pages: int, hot_blocks_per_request: int, tail_pages: int = 1):
        self.cfg = _Config(page_size, num_blocks, num_host_blocks, max_requests, max_pages,
                           hot_blocks_per_request, tail_pages)
        h = ctypes.c_void_p()
        self._check(lib().hs_policy_create(ctypes.byref(self.cfg), ctypes.byref(h)), "create")
        self.h = h
        cap = max(64, 2 * num_blocks + 2 * max_requests * max_pages)
        self._bufs = {k: np.zeros((cap, 3), np.int32) for k in ("bt", "hbt", "hot")}
        self._reset = np.zeros(max(1, max_requests), np.int32)
        self._off = np.zeros((cap, 2), np.int32)
        self._cap = cap

    @staticmethod
    def _check(status: int, what: str) -> None:
        if status != OK:
            raise PolicyError(status, f"hs_policy_{what} failed")

    def _edits(self) -> _Edits:
        b = self._bufs
        return _Edits(b["bt"].ctypes.data, 0, self._cap, b["hbt"].ctypes.data, 0, self._cap,
                      b["hot"].ctypes.data, 0, self._cap, self._reset.ctypes.data, 0,
                      self._reset.size, self._off.ctypes.data, 0, self._cap, 0, 0, 0)

    def _out(self, e: _Edits) -> Edits:
        b = self._bufs
        return Edits(b["bt"][:e.n_bt].copy(), b["hbt"][:e.n_hbt].copy(), b["hot"][:e.n_hot].copy(),
                     self._reset[:e.n_reset].copy(), self._off[:e.n_offload].copy(), e.evicted,
                     e.leased, e.returned)

    def admit(self, req: int, ctx_len: int, host_block_of_page=None,
              resident_prefix: bool = False) -> Edits:
        hb = None if host_block_of_page is None else np.ascontiguousarray(host_block_of_page,
                                                                          np.int32)
        e = self._edits()
        self._check(lib().hs_policy_admit(self.h, req, ctx_len, None if hb is None else hb.ctypes.data,
                                          int(resident_prefix), ctypes.byref(e)), "admit")
        return self._out(e)

    def finish(self, req: int) -> Edits:
        e = self._edits()
        self._check(lib().hs_policy_finish(self.h, req, ctypes.byref(e)), "finish")
        return self._out(e)

    def step(self, stamp: int, reqs, ctx_lens, topk=None) -> Edits:
        r = np.ascontiguousarray(reqs, np.int32)
        c = np.ascontiguousarray(ctx_lens, np.int32)
        t = None if topk is None else np.ascontiguousarray(topk, np.int32).reshape(r.size, -1)
        k = 0 if t is None else t.shape[1]
        e = self._edits()
        self._check(lib().hs_policy_step(self.h, stamp, r.ctypes.data, c.ctypes.data, r.size,
                                         None if t is None else t.ctypes.data, k,
                                         ctypes.byref(e)), "step")
        return self._out(e)

    def step_pages(self, reqs, ctx_lens, page_use=None) -> Edits:
        """A step with coldness given per page: page_use uint32 [n, stride]
        (row i for reqs[i]), e.g. hs_page_touch's table copied to host."""
        r = np.ascontiguousarray(reqs, np.int32)
        c = np.ascontiguousarray(ctx_lens, np.int32)
        u = None if page_use is None else np.ascontiguousarray(page_use, np.uint32)
        if u is not None and u.shape[0] != r.size:
            raise ValueError("page_use needs one row per request")
        stride = 0 if u is None else u.shape[1]
        e = self._edits()
        self._check(lib().hs_policy_step_pages(self.h, r.ctypes.data, c.ctypes.data, r.size,
                                               None if u is None else u.ctypes.data, stride,
                                               ctypes.byref(e)), "step_pages")
        return self._out(e)

    def tables(self, req: int):
        mp, hb = self.cfg.max_pages, self.cfg.hot_blocks_per_request
        bt, hbt, hot = (np.zeros(mp, np.int32), np.zeros(mp, np.int32), np.zeros(hb, np.int32))
        self._check(lib().hs_policy_tables(self.h, req, bt.ctypes.data, hbt.ctypes.data,
                                           hot.ctypes.data), "tables")
        return bt, hbt, hot

    def free_blocks(self) -> int:
        return lib().hs_policy_free_blocks(self.h)

    def close(self) -> None:
        if getattr(self, "h", None):
            lib().hs_policy_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
