"""GPU parity of hs_page_touch (page coldness stamps) with the oracle, bit
for bit, and the residency policy driven by the stamps the GPU writes making
the same decisions as the policy reading the lists."""

from __future__ import annotations

import os
import zlib

import numpy as np
import pytest
import torch

import hs_gen
import oracle
from harness import policy_workload
from test_policy import PageUseDecider, _same_edits

pytestmark = pytest.mark.gpu

PAGE = hs_gen.PAGE


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import serving_memory_tier_amd as hs
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hs.lib()


def _gpu_touch(ctx, topk, stamp, use, entries=None, page=PAGE):
    """hs_page_touch on device copies of the inputs; use is updated in place."""
    import serving_memory_tier_amd as hs
    R, mp = use.shape
    c = torch.from_numpy(np.ascontiguousarray(ctx, np.int32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(topk, np.int32).reshape(R, -1)).cuda()
    u = torch.from_numpy(use).cuda()
    E = t.shape[1] if entries is None else entries
    lay = hs.layout_of(page, hs_gen.ROW_BYTES, 1, max(512, page), page, 0)
    batch = hs.HsBatch(R, mp, None, None, None, None, c.data_ptr(), None, None, None)
    print(f"[touch] R={R} max_pages={mp} entries={E} stamp={stamp}", flush=True)
    hs.hs_page_touch(lay, batch, t if t.numel() else None, E, stamp, u)
    torch.cuda.synchronize()
    use[:] = u.cpu().numpy()


CASES = {  # name: (R, max_pages, entries per request)
    "one_entry": (3, 10, 1),
    "ragged_small": (7, 50, 5),
    "one_block_minus_one": (4, 30, 1023),
    "one_block": (4, 30, 1024),
    "one_block_plus_one": (4, 30, 1025),
    "ragged_many_blocks": (9, 200, 3000),
    "multi_layer_lists": (64, 2300, 16 * 2048),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_page_touch_matches_oracle(name):
    R, mp, E = CASES[name]
    rs = np.random.default_rng(zlib.crc32(name.encode()))
    ctx = rs.integers(1, (mp + 5) * PAGE, size=R).astype(np.int32)  # some beyond the table
    topk = rs.integers(-3, (mp + 6) * PAGE, size=(R, E)).astype(np.int32)
    topk[:, 0] = ctx - 1
    if E > 1:
        topk[:, -1] = ctx
    use0 = rs.integers(0, 1 << 32, size=(R, mp), dtype=np.uint64).astype(np.uint32)
    exp = use0.copy()
    oracle.page_touch(ctx, topk, 0xFFFFFFF0, exp)
    got = use0.copy()
    _gpu_touch(ctx, topk, 0xFFFFFFF0, got)
    assert np.array_equal(got, exp)
    assert not np.array_equal(got, use0)


@pytest.mark.parametrize("seed", list(range(12)))
def test_page_touch_sweep(seed):
    """Random page sizes (1 to 4096 tokens), batches, table lengths and list
    lengths (0 to 5000), stamps anywhere in 32 bits."""
    rs = np.random.default_rng(3000 + seed)
    page = int(rs.choice([1, 16, 64, 256, 4096]))
    R = int(rs.integers(1, 41))
    mp = int(rs.integers(1, 501))
    E = int(rs.integers(0, 5001))
    ctx = rs.integers(1, (mp + 3) * page + 1, size=R).astype(np.int32)
    topk = rs.integers(-3, (mp + 4) * page, size=(R, E)).astype(np.int32)
    use0 = rs.integers(0, 1 << 32, size=(R, mp), dtype=np.uint64).astype(np.uint32)
    stamp = int(rs.integers(1, 1 << 32, dtype=np.uint64))
    exp = use0.copy()
    oracle.page_touch(ctx, topk, stamp, exp, page=page)
    got = use0.copy()
    _gpu_touch(ctx, topk, stamp, got, page=page)
    assert np.array_equal(got, exp)


def test_page_touch_with_nothing_to_do_changes_nothing():
    use0 = np.arange(12, dtype=np.uint32).reshape(3, 4)
    got = use0.copy()
    _gpu_touch(np.array([100, 100, 100], np.int32), np.zeros((3, 0), np.int32), 7, got)
    assert np.array_equal(got, use0)


@pytest.mark.parametrize("group", [1, 2])
def test_gpu_page_stamps_drive_the_policy(group):
    """The policy workload rebuilt with a decider whose coldness comes from
    hs_page_touch on the GPU (checked against the oracle on every call)
    makes exactly the edits of the policy that reads the lists."""
    wl, dec = policy_workload(group=group, L=2 * group)
    calls = []

    def touch(ctx, topk, stamp, use):
        exp = use.copy()
        oracle.page_touch(ctx, topk, stamp, exp)
        _gpu_touch(ctx, topk, stamp, use)
        assert np.array_equal(use, exp), f"page stamps, stamp {stamp}"
        calls.append(stamp)

    d = PageUseDecider(wl.R, wl.n_blocks, dec.p.cfg.num_host_blocks, dec.p.cfg.max_pages, wl.C,
                       dec.p.cfg.tail_pages, touch)
    spec = hs_gen.Spec(name=wl.name, seed=wl.seed, R=wl.R, L=wl.L, K=wl.K, C=wl.C,
                       steps=len(wl.steps), ctx0=wl.ctx0.astype(np.int64), classes=wl.classes,
                       append=int(wl.steps[0].ctx[0] - wl.ctx0[0]), group=group)
    wl2 = hs_gen.build_dynamic(spec, d, wl.n_blocks, dec.p.cfg.num_host_blocks)
    assert len(calls) == len(wl.steps) - 1
    _same_edits(wl, wl2)
