"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/hisparse.h declares, and rejects bad arguments with the
documented status codes before touching the GPU."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import serving_memory_tier_amd as hs
from serving_memory_tier_amd._lib import HsBatch, HsLayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    return hs.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    return sorted(set(re.findall(r"^\s*(?:hs_status|const char\*|size_t)\s+(hs_\w+)\s*\(", text,
                                 re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(hs.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert hs.hs_status_string(0) == "ok"
    assert "invalid" in hs.hs_status_string(1)
    assert "unsupported" in hs.hs_status_string(2)
    assert "launch" in hs.hs_status_string(3)
    assert "unknown" in hs.hs_status_string(99)
    assert lib.hs_last_error() == b""           # no HIP failure on this thread yet


def _layout(**kw):
    d = dict(page_size=64, row_bytes=656, num_layers=1, hot_capacity=4096, pool_rows=64 * 100,
             host_rows=64 * 100)
    d.update(kw)
    lay = HsLayout(d["page_size"], d["row_bytes"], d["num_layers"], d["hot_capacity"],
                   d["pool_rows"], d["host_rows"], d["pool_rows"] * d["row_bytes"],
                   d["host_rows"] * d["row_bytes"])
    for k in ("pool_layer_stride", "host_layer_stride"):
        if k in kw:
            setattr(lay, k, kw[k])
    return lay


def _batch(R=2):
    fake = 0x1000  # never dereferenced: every call below fails validation first
    return HsBatch(R, 16, fake, fake, fake, fake, fake, fake, fake, fake)


def _resolve(lib, lay, bat, topk=0x1000, K=2048, stamp=1, rows=0x1000, stats=0x1000):
    return lib.hs_resolve(ctypes.byref(lay) if lay is not None else None,
                          ctypes.byref(bat) if bat is not None else None, topk, K,
                          ctypes.c_uint32(stamp), rows, None, stats, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=48), 1), (dict(page_size=0), 1), (dict(page_size=8192), 1),
    (dict(row_bytes=650), 1), (dict(row_bytes=0), 1), (dict(num_layers=0), 1),
    (dict(row_bytes=4096 + 16), 2),
    (dict(hot_capacity=100), 1), (dict(hot_capacity=0), 1), (dict(hot_capacity=16384), 2),
    (dict(hot_capacity=12288 + 64), 2),
    (dict(pool_rows=0), 1), (dict(pool_rows=100), 1), (dict(host_rows=-64), 1),
    (dict(pool_rows=1 << 31), 1),
    (dict(num_layers=2, pool_layer_stride=10), 1),
    (dict(num_layers=2, pool_layer_stride=64 * 100 * 656 + 8), 1),
    (dict(num_layers=2, host_layer_stride=64 * 100 * 656 + 24), 1),
])
def test_resolve_rejects_bad_layout(lib, kw, code):
    assert _resolve(lib, _layout(**kw), _batch()) == code


def test_rejects_misaligned_buffers(lib):
    lay = _layout()
    b = _batch()
    b.kv_pool = 0x1008
    assert _resolve(lib, lay, b) == 1
    b = _batch()
    b.host_pool = 0x1004
    assert _resolve(lib, lay, b) == 1
    ok = _batch()
    r = lambda out: lib.hs_resolve(ctypes.byref(lay), ctypes.byref(ok), 0x1000, 2048,
                                   ctypes.c_uint32(1), 0x1000, out, 0x1000, None)
    assert r(0x1008) == 1
    assert lib.hs_gather(ctypes.byref(lay), 0x1008, 0x1000, 2, 16, 0x1000, None) == 1
    assert lib.hs_gather(ctypes.byref(lay), 0x1000, 0x1000, 2, 16, 0x1001, None) == 1
    assert lib.hs_offload_prefix_pages(ctypes.byref(lay), 0x1000, 0x1004, 0x1000, 3, None) == 1


def test_resolve_rejects_bad_call(lib):
    lay = _layout()
    assert _resolve(lib, None, _batch()) == 1
    assert _resolve(lib, lay, None) == 1
    assert _resolve(lib, lay, _batch(), topk=None) == 1
    assert _resolve(lib, lay, _batch(), rows=None) == 1
    assert _resolve(lib, lay, _batch(), stats=None) == 1
    assert _resolve(lib, lay, _batch(), stamp=0) == 1
    assert _resolve(lib, lay, _batch(), K=0) == 1
    assert _resolve(lib, lay, _batch(), K=8193) == 2
    bad = _batch()
    bad.kv_pool = None
    assert _resolve(lib, lay, bad) == 1
    bad = _batch()
    bad.max_pages = 0
    assert _resolve(lib, lay, bad) == 1
    bad = _batch(R=-1)
    assert _resolve(lib, lay, bad) == 1
    # fill_sync: words without a pointer, a pointer with too few words
    bad = _batch()
    bad.fill_sync_words = 64
    assert _resolve(lib, lay, bad) == 1
    bad = _batch()
    bad.fill_sync = 0x1000
    bad.fill_sync_words = 63
    assert _resolve(lib, lay, bad) == 1
    bad.fill_sync_words = -1
    assert _resolve(lib, lay, bad) == 1


def test_plan_rejects_bad_call(lib):
    lay, bat = _layout(), _batch()
    f = lambda P, K, pairs, n: lib.hs_plan_replay(ctypes.byref(lay), ctypes.byref(bat), 0x1000,
                                                  P, K, ctypes.c_uint32(1), 0x1000, None, 0x1000,
                                                  pairs, n, None)
    assert f(0, 2048, None, 0) == 1
    assert f(5, 2048, None, 0) == 2      # 10240 entries > 8192
    assert f(4, 2048, None, -1) == 1
    assert f(4, 2048, None, 3) == 1      # pairs missing


def test_grouped_rejects_bad_call(lib):
    lay, bat = _layout(num_layers=4), _batch()
    g = lambda G, K=2048: lib.hs_resolve_grouped(ctypes.byref(lay), ctypes.byref(bat), G, 0x1000,
                                                 1, K, ctypes.c_uint32(1), 0x1000, None, 0x1000,
                                                 None, 0, None)
    assert g(3) == 1       # 3 does not divide 4 layers
    assert g(0) == 1
    assert g(-2) == 1
    assert g(2, K=0) == 1
    assert g(2, K=8193) == 2


def test_stages_reject_bad_call(lib):
    lay, bat = _layout(), _batch()
    L, B = ctypes.byref(lay), ctypes.byref(bat)
    fetch = lambda topk, P, K, out: lib.hs_resolve_fetch(L, B, topk, P, K, out, None)
    assert fetch(0x1000, 1, 2048, None) == 1          # the prefetch writes into gather_out
    assert fetch(None, 1, 2048, 0x1000) == 1
    assert fetch(0x1000, 0, 2048, 0x1000) == 1
    assert fetch(0x1000, 5, 2048, 0x1000) == 2
    move = lambda rows: lib.hs_resolve_move(L, B, 0x1000, 1, 2048, rows, None, None)
    assert move(None) == 1
    commit = lambda rows, out: lib.hs_resolve_commit(L, B, 0x1000, 1, 2048, rows, out, None)
    assert commit(0x1000, None) == 1
    assert commit(None, 0x1000) == 1
    dec = lambda stamp, stats: lib.hs_resolve_decide(L, B, 0x1000, 1, 2048, ctypes.c_uint32(stamp),
                                                     0x1000, None, stats, None)
    assert dec(0, 0x1000) == 1
    assert dec(1, None) == 1
    empty = _batch(R=0)
    E = ctypes.byref(empty)
    assert lib.hs_resolve_fetch(L, E, 0x1000, 1, 2048, 0x1000, None) == 0   # nothing to do
    assert lib.hs_resolve_commit(L, E, 0x1000, 1, 2048, 0x1000, 0x1000, None) == 0


def test_gather_and_offload_reject(lib):
    lay = _layout()
    g = lambda pool, rows, R, n, out: lib.hs_gather(ctypes.byref(lay), pool, rows, R, n, out, None)
    assert g(None, 0x1000, 1, 10, 0x1000) == 1
    assert g(0x1000, None, 1, 10, 0x1000) == 1
    assert g(0x1000, 0x1000, 1, 10, None) == 1
    assert g(0x1000, 0x1000, -1, 10, 0x1000) == 1
    assert g(0x1000, 0x1000, 1 << 20, 100_000, 0x1000) == 2  # more than 2^31 wave chunks
    assert g(0x1000, 0x1000, 0, 10, 0x1000) == 0            # nothing to do
    o = lambda pool, host, pairs, n: lib.hs_offload_prefix_pages(ctypes.byref(lay), pool, host,
                                                                pairs, n, None)
    assert o(0x1000, 0x1000, 0x1000, -1) == 1
    assert o(None, 0x1000, 0x1000, 1) == 1
    assert o(0x1000, None, 0x1000, 1) == 1
    assert o(0x1000, 0x1000, None, 1) == 1
    assert o(0x1000, 0x1000, None, 0) == 0                  # nothing to do


def test_host_alloc_rejects(lib):
    p = ctypes.c_void_p()
    assert lib.hs_host_alloc(0, ctypes.byref(p)) == 1
    assert lib.hs_host_alloc(64, None) == 1
    assert lib.hs_host_free(None) == 0
    assert lib.hs_host_device_pointer(None, ctypes.byref(p)) == 1


def test_page_touch_rejects(lib):
    lay = _layout()
    b = HsBatch(4, 16, None, None, None, None, 0x1000, None, None, None)
    t = lambda lay_, bat, topk, E, use: lib.hs_page_touch(
        ctypes.byref(lay_) if lay_ is not None else None,
        ctypes.byref(bat) if bat is not None else None, topk, E, 5, use, None)
    assert t(None, b, 0x1000, 8, 0x1000) == 1
    assert t(lay, None, 0x1000, 8, 0x1000) == 1
    assert t(lay, b, None, 8, 0x1000) == 1
    assert t(lay, b, 0x1000, 8, None) == 1
    assert t(lay, b, 0x1000, -1, 0x1000) == 1
    assert t(lay, b, 0x1000, 1024 * 65535 + 1, 0x1000) == 2
    nb = HsBatch(4, 16, None, None, None, None, None, None, None, None)
    assert t(lay, nb, 0x1000, 8, 0x1000) == 1                # no context lengths
    bad = HsBatch(4, 0, None, None, None, None, 0x1000, None, None, None)
    assert t(lay, bad, 0x1000, 8, 0x1000) == 1               # no table columns
    assert t(lay, b, None, 0, None) == 0                     # nothing to do
    empty = HsBatch(0, 16, None, None, None, None, None, None, None, None)
    assert t(lay, empty, None, 8, None) == 0


def test_sparse_mla_rejects(lib):
    lay = _layout()
    P = 0x1000
    f = lambda lay_, kv, ids, T, K, q, H, out, lse, ws, wsb: lib.hs_sparse_mla_decode(
        ctypes.byref(lay_), kv, ids, T, K, q, H, 0.1, out, lse, ws, wsb, None)
    need = lib.hs_sparse_mla_workspace_bytes(32, 128, 2048)
    assert need > 0
    assert f(_layout(row_bytes=512), P, P, 1, 64, P, 16, P, P, P, need) == 2
    assert f(lay, P, P, 1, 64, P, 24, P, P, P, need) == 1        # heads not a multiple of 16
    assert f(lay, P, P, 1, 64, P, 0, P, P, P, need) == 1
    assert f(lay, P, P, -1, 64, P, 16, P, P, P, need) == 1
    assert f(lay, P, P, 70000, 64, P, 16, P, P, P, need) == 2
    assert f(lay, None, P, 1, 64, P, 16, P, P, P, need) == 1
    assert f(lay, P, None, 1, 64, P, 16, P, P, P, need) == 1
    assert f(lay, P, P, 1, 64, None, 16, P, P, P, need) == 1
    assert f(lay, P, P, 1, 64, P + 4, 16, P, P, P, need) == 1    # misaligned queries
    assert f(lay, P, P, 32, 2048, P, 128, P, P, None, need) == 1  # workspace needed
    assert f(lay, P, P, 32, 2048, P, 128, P, P, P, need - 16) == 1
    assert f(lay, P, P, 1, 64 * 2048 + 1, P, 16, P, P, P, 1 << 40) == 2   # top_k over the bound
    assert f(lay, P, P, 0, 64, None, 16, None, None, None, 0) == 0   # nothing to do
    assert lib.hs_sparse_mla_workspace_bytes(0, 16, 64) == 0


def test_sparse_mla_noalloc_rejects(lib):
    """The allocation-free form checks like hs_sparse_mla_decode and refuses,
    before any GPU work, sizes whose workspace exceeds its per-device array."""
    lay = _layout()
    P = 0x1000
    f = lambda lay_, kv, ids, T, K, q, H, out, lse: lib.hs_sparse_mla_decode_noalloc(
        ctypes.byref(lay_), kv, ids, T, K, q, H, 0.1, out, lse, None)
    cap = lib.hs_sparse_mla_noalloc_max_workspace()
    assert cap == hs.hs_sparse_mla_noalloc_max_workspace() == 64 << 20
    assert lib.hs_sparse_mla_workspace_bytes(32, 128, 2048) <= cap    # the decode shape fits
    assert lib.hs_sparse_mla_workspace_bytes(16, 128, 131072) > cap  # 64 key splits
    assert f(lay, P, P, 16, 131072, P, 128, P, P) == 2               # beyond the array
    assert f(_layout(row_bytes=512), P, P, 1, 64, P, 16, P, P) == 2
    assert f(lay, P, P, 1, 64, P, 24, P, P) == 1
    assert f(lay, None, P, 1, 64, P, 16, P, P) == 1
    assert f(lay, P, P, 1, 64, P + 4, 16, P, P) == 1
    assert f(lay, P, P, 0, 64, None, 16, None, None) == 0            # nothing to do
