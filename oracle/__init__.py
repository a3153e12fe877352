"""CPU oracle for the top-K resolver, row gather, prefix-page offload and page
coldness stamps.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It wraps the plain
C++ statement of the method in ``hisparse_oracle.cpp`` (built with g++, no GPU
code, nothing shared with the HIP library) for numpy arrays.

Every function here mutates the arrays it is given exactly as the GPU library
mutates its device buffers, so a test can run both on equal copies and compare.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hisparse_oracle.cpp")
# HS_ORACLE_LIB points the wrapper at another build of the oracle source: the
# mutation tests use it to check that the pins catch planted mistakes.
LIB = os.environ.get("HS_ORACLE_LIB") or os.path.join(HERE, "libhisparse_oracle.so")

PAGE = 64
ROW_BYTES = 656

_lib = None


def build() -> str:
    """Compile the oracle (always; callers decide when a rebuild is wanted)."""
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-shared", "-fPIC",
                    "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        i32, i64, u32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
        lib.oracle_gather.argtypes = [i32, i32, i64, i64, i32, i32, i32, vp, vp, vp]
        lib.oracle_offload.argtypes = [i32, i32, i32, i64, i64, i64, i64, vp, vp, vp, i32]
        lib.oracle_resolve.argtypes = [i32, i32, i32, i32, i64, i64, i64, i64, i32, i32, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, i32, u32, vp, vp, vp]
        lib.oracle_resolve_grouped.argtypes = [i32, i32, i32, i32, i32, i64, i64, i64, i64, i32,
                                               i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, u32,
                                               vp, vp, vp]
        lib.oracle_page_touch.argtypes = [i32, i32, i32, i32, vp, vp, u32, vp]
        for f in (lib.oracle_gather, lib.oracle_offload, lib.oracle_resolve,
                  lib.oracle_resolve_grouped, lib.oracle_page_touch):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data


def _check(a: np.ndarray, dtype, name: str):
    if a.dtype != dtype:
        raise TypeError(f"{name} must be {np.dtype(dtype).name}, got {a.dtype}")


def gather(pool: np.ndarray, rows: np.ndarray, page: int = PAGE) -> np.ndarray:
    """out[r, l, i] = pool[l, rows[r, l, i]] (zero row outside the pool).

    pool: uint8 [L, pool_rows, 656]; rows: int32 [R, L, N] -> uint8 [R, L, N, 656].
    """
    _check(pool, np.uint8, "pool")
    _check(rows, np.int32, "rows")
    L, pool_rows, rb = pool.shape
    R, L2, N = rows.shape
    assert L2 == L and rb % 16 == 0
    out = np.empty((R, L, N, rb), dtype=np.uint8)
    _load().oracle_gather(page, rb, pool_rows, pool_rows * rb, R, L, N, _ptr(pool), _ptr(rows),
                          _ptr(out))
    return out


def offload(pool: np.ndarray, host: np.ndarray, pairs: np.ndarray, page: int = PAGE) -> None:
    """host[l, hb page] = pool[l, db page] for each (db, hb) pair and every layer."""
    _check(pool, np.uint8, "pool")
    _check(host, np.uint8, "host")
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    L, pool_rows, rb = pool.shape
    L2, host_rows, rb2 = host.shape
    assert L2 == L and rb == rb2 and rb % 16 == 0
    _load().oracle_offload(page, rb, L, pool_rows, pool_rows * rb, host_rows, host_rows * rb,
                           _ptr(pool), _ptr(host), _ptr(pairs), pairs.shape[0])


def page_touch(ctx_len: np.ndarray, topk: np.ndarray, stamp: int, page_use: np.ndarray,
               page: int = PAGE) -> None:
    """Page coldness in place: page_use[r, t // page] = stamp for every entry t
    of topk[r] (any shape [R, ...], flattened per request) with 0 <= t < ctx_len[r]
    and t // page < max_pages.  page_use: uint32 [R, max_pages]."""
    _check(page_use, np.uint32, "page_use")
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    R, max_pages = page_use.shape
    t = np.ascontiguousarray(topk, dtype=np.int32).reshape(R, -1)
    assert ctx.shape == (R,)
    _load().oracle_page_touch(page, R, max_pages, t.shape[1], _ptr(ctx), _ptr(t), stamp,
                              _ptr(page_use))


def resolve(pool: np.ndarray, host: np.ndarray, block_table: np.ndarray,
            host_block_table: np.ndarray, ctx_len: np.ndarray, hot_blocks: np.ndarray,
            slot_token: np.ndarray, slot_stamp: np.ndarray, topk: np.ndarray, stamp: int,
            gather_out: bool = True, page: int = PAGE):
    """Resolve one batch in place; returns (rows, stats, out-or-None).

    pool uint8 [L, pool_rows, 656] (hot slots written); host uint8 [L, host_rows, 656];
    block_table / host_block_table int32 [R, max_pages]; ctx_len int32 [R];
    hot_blocks int32 [R, C/64]; slot_token int32 / slot_stamp uint32 [R, L, C] (updated);
    topk int32 [R, L, N] or [R, L, P, K] (a plan over P positions).
    rows has the shape of topk; stats is int32 [R, L, 8] =
    (resident, hit, miss, overflow, invalid, pad, dup, 0).
    """
    for a, t, n in ((pool, np.uint8, "pool"), (host, np.uint8, "host"),
                    (block_table, np.int32, "block_table"),
                    (host_block_table, np.int32, "host_block_table"),
                    (ctx_len, np.int32, "ctx_len"), (hot_blocks, np.int32, "hot_blocks"),
                    (slot_token, np.int32, "slot_token"), (slot_stamp, np.uint32, "slot_stamp"),
                    (topk, np.int32, "topk")):
        _check(a, t, n)
    L, pool_rows, rb = pool.shape
    host_rows = host.shape[1]
    R, max_pages = block_table.shape
    C = slot_token.shape[2]
    assert slot_token.shape == slot_stamp.shape == (R, L, C)
    assert hot_blocks.shape == (R, C // page)
    N = int(np.prod(topk.shape[2:]))
    assert topk.shape[:2] == (R, L)
    rows = np.empty(topk.shape, dtype=np.int32)
    stats = np.zeros((R, L, 8), dtype=np.int32)
    out = np.empty(topk.shape + (rb,), dtype=np.uint8) if gather_out else None
    topk_c = np.ascontiguousarray(topk)
    _load().oracle_resolve(page, rb, L, C, pool_rows, pool_rows * rb, host_rows, host_rows * rb,
                           R, max_pages, _ptr(pool), _ptr(host), _ptr(block_table),
                           _ptr(host_block_table), _ptr(ctx_len), _ptr(hot_blocks),
                           _ptr(slot_token), _ptr(slot_stamp), _ptr(topk_c), N,
                           ctypes.c_uint32(stamp), _ptr(rows), _ptr(stats), _ptr(out))
    return rows, stats, out


def plan_replay(pool, host, block_table, host_block_table, ctx_len, hot_blocks, slot_token,
                slot_stamp, topk, stamp, gather_out=True, offload_pairs=None, page=PAGE):
    """A per-step plan over P query positions: resolve of the concatenated
    position lists with one stamp commit, then (optionally) the prefix offload."""
    res = resolve(pool, host, block_table, host_block_table, ctx_len, hot_blocks, slot_token,
                  slot_stamp, topk, stamp, gather_out, page)
    if offload_pairs is not None and len(offload_pairs):
        offload(pool, host, offload_pairs, page)
    return res


def resolve_grouped(pool: np.ndarray, host: np.ndarray, block_table: np.ndarray,
                    host_block_table: np.ndarray, ctx_len: np.ndarray, hot_blocks: np.ndarray,
                    slot_token: np.ndarray, slot_stamp: np.ndarray, topk: np.ndarray, stamp: int,
                    group: int, gather_out: bool = True, page: int = PAGE):
    """Grouped resolve ("Use sparsity when needed": IndexShare, one indexer
    layer per group of sparse-MLA layers): the pool's L layers form L / group
    groups that share one top-K list and one hot-buffer state.  Decisions are
    made once per group; each copy is made in every layer of the group; every
    layer gets the group's row ids.

    slot_token / slot_stamp [R, L/group, C] (updated); topk [R, L/group, N] or
    [R, L/group, P, K]; rows / stats per group; out [R, L, ...topk dims, 656].
    Returns (rows, stats, out-or-None).
    """
    for a, t, n in ((pool, np.uint8, "pool"), (host, np.uint8, "host"),
                    (block_table, np.int32, "block_table"),
                    (host_block_table, np.int32, "host_block_table"),
                    (ctx_len, np.int32, "ctx_len"), (hot_blocks, np.int32, "hot_blocks"),
                    (slot_token, np.int32, "slot_token"), (slot_stamp, np.uint32, "slot_stamp"),
                    (topk, np.int32, "topk")):
        _check(a, t, n)
    L, pool_rows, rb = pool.shape
    assert group >= 1 and L % group == 0
    NG = L // group
    host_rows = host.shape[1]
    R, max_pages = block_table.shape
    C = slot_token.shape[2]
    assert slot_token.shape == slot_stamp.shape == (R, NG, C)
    assert hot_blocks.shape == (R, C // page)
    assert topk.shape[:2] == (R, NG)
    N = int(np.prod(topk.shape[2:]))
    rows = np.empty(topk.shape, dtype=np.int32)
    stats = np.zeros((R, NG, 8), dtype=np.int32)
    out = (np.empty((R, L) + topk.shape[2:] + (rb,), dtype=np.uint8) if gather_out else None)
    topk_c = np.ascontiguousarray(topk)
    rc = _load().oracle_resolve_grouped(page, rb, L, group, C, pool_rows, pool_rows * rb,
                                        host_rows, host_rows * rb, R, max_pages, _ptr(pool),
                                        _ptr(host), _ptr(block_table), _ptr(host_block_table),
                                        _ptr(ctx_len), _ptr(hot_blocks), _ptr(slot_token),
                                        _ptr(slot_stamp), _ptr(topk_c), N, ctypes.c_uint32(stamp),
                                        _ptr(rows), _ptr(stats), _ptr(out))
    assert rc == 0
    return rows, stats, out
