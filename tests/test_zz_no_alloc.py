"""The allocation-free sparse MLA decode (hs_sparse_mla_decode_noalloc)
through the C ABI against hs_sparse_mla_decode with a caller workspace: the
same kernels, so the outputs must be identical bit for bit.  Two calls in a
row share the library's per-device workspace, the second with a smaller
input, and both are also checked against the float64 oracle within the
tolerance the arithmetic fixes (2^-8 max|v| + 1e-6 on out, 1e-4 on lse).
Runs last: it must pass alone in a fresh process and after every other test."""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from oracle import sparse_mla as sm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import serving_memory_tier_amd as hs
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hs.lib()


def _inputs(rs, n_rows, T, H, K):
    sign = rs.integers(0, 2, size=(n_rows, 512)) << 7
    e = rs.integers(0, 9, size=(n_rows, 512)) << 3
    m = rs.integers(0, 8, size=(n_rows, 512))
    pool = np.zeros((n_rows, 656), np.uint8)
    pool[:, :512] = (sign | e | m).astype(np.uint8)
    pool[:, 512:528] = rs.uniform(0.05, 0.3, size=(n_rows, 4)).astype("<f4").view(np.uint8)
    rope = rs.standard_normal((n_rows, 64)).astype(np.float32).view(np.uint32) >> 16
    pool[:, 528:] = rope.astype("<u2").view(np.uint8)
    ids = rs.integers(0, n_rows, size=(T, K)).astype(np.int32)
    ids[0, :5] = [-1, n_rows, 3, 3, -7]            # nothing, out of the pool, a duplicate
    q = (rs.standard_normal((T, H, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return pool, ids, q


def _both(pool, ids, q, sm_scale):
    import serving_memory_tier_amd as hs
    T, K = ids.shape
    H = q.shape[1]
    lay = hs.layout_of(1, 656, 1, 64, pool.shape[0], 0)
    gp = torch.from_numpy(pool).cuda()
    gi = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
    gq = torch.from_numpy(q.view(np.int16)).cuda()
    res = []
    for noalloc in (True, False):
        out = torch.full((T, H, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            hs.hs_sparse_mla_decode_noalloc(lay, gp, gi, T, K, gq, H, sm_scale, out, lse)
        else:
            wsb = hs.hs_sparse_mla_workspace_bytes(T, H, K)
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
            hs.hs_sparse_mla_decode(lay, gp, gi, T, K, gq, H, sm_scale, out, lse, ws, wsb)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


def test_noalloc_equals_workspace_form_twice():
    import serving_memory_tier_amd as hs
    rs = np.random.default_rng(77)
    cap = hs.hs_sparse_mla_noalloc_max_workspace()
    # the decode shape (32 tokens x 128 heads x 2048 rows), then a smaller call
    for T, H, K in ((32, 128, 2048), (5, 48, 700)):
        need = hs.hs_sparse_mla_workspace_bytes(T, H, K)
        assert 0 < need <= cap
        print(f"[noalloc] T={T} H={H} K={K} workspace {need} of {cap}", flush=True)
        pool, ids, q = _inputs(rs, 6000, T, H, K)
        (o1, l1), (o2, l2) = _both(pool, ids, q, 0.0417)
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), "out differs"
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "lse differs"
        ref_out, ref_lse = sm.sparse_mla_decode(pool, ids, q, 0.0417)
        _, v_all = sm.decode_rows(pool)
        vmax = np.abs(v_all).max()
        assert np.abs(o1 - ref_out).max() <= 2.0 ** -8 * vmax + 1e-6
        assert np.abs(l1 - ref_lse).max() <= 1e-4


def test_noalloc_rejects_beyond_its_workspace():
    import serving_memory_tier_amd as hs
    lay = hs.layout_of(1, 656, 1, 64, 64, 0)
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(hs.HsError) as e:
        # 16 tokens x 128 heads x 131,072 rows: 64 key splits, beyond the array
        assert hs.hs_sparse_mla_workspace_bytes(16, 128, 131072) > \
            hs.hs_sparse_mla_noalloc_max_workspace()
        hs.hs_sparse_mla_decode_noalloc(lay, t, t, 16, 131072, t, 128, 0.1, t, t)
    assert e.value.status == hs.HS_ERR_UNSUPPORTED
