"""GPU parity on hand-made and randomised edge cases, through the C ABI.

Covers what the synthetic workloads do not: the hand-worked example (4-token
pages, 8 slots), padding, duplicates, out-of-range tokens, null pages without
host copies, table entries pointing outside the pools, unusable hot blocks,
non-monotone stamps, ragged and maximal list sizes, maximal hot capacity,
other page sizes and row sizes, an empty batch, and the gather and offload
entry points on their own.  The randomised cases run each path of the
library: the one-call form, the serial stages and the caller-scheduled
overlapped stages.
"""

from __future__ import annotations

import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import stages
from harness import run_tiny, tiny_instance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import serving_memory_tier_amd as hs
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available()
    hs.lib()


def _say(msg):
    print(msg, flush=True)


class GpuCase:
    """One batch in device memory, built from the same numpy arrays the oracle gets."""

    def __init__(self, page, pool, host, bt, hbt, ctx, hot, tok, stp, C, fill_sync=False,
                 pad=0):
        import serving_memory_tier_amd as hs
        self.hs = hs
        L, pool_rows, rb = pool.shape
        host_rows = host.shape[1]
        self.page, self.rb, self.L, self.C = page, rb, L, C
        # pad > 0: every layer of both pools is followed by `pad` bytes of
        # 0xA5 that no call may touch (layer strides past the rows)
        self.pad = pad
        ps, hs_ = pool_rows * rb + pad, host_rows * rb + pad
        self.pool_flat = torch.full((L * ps,), 0xA5, dtype=torch.uint8, device="cuda")
        self.pool = torch.as_strided(self.pool_flat, (L, pool_rows, rb), (ps, rb, 1))
        self.pool.copy_(torch.from_numpy(pool))
        self.host_pool = hs.HostPool(max(1, L * hs_))
        self.host_flat = self.host_pool.tensor[:L * hs_]
        self.host_flat.fill_(0xA5)
        self.host = torch.as_strided(self.host_flat, (L, host_rows, rb), (hs_, rb, 1))
        self.host.copy_(torch.from_numpy(host))
        self.bt = torch.from_numpy(bt).cuda()
        self.hbt = torch.from_numpy(hbt).cuda()
        self.ctx = torch.from_numpy(ctx).cuda()
        self.hot = torch.from_numpy(hot).cuda()
        self.tok = torch.from_numpy(tok).cuda()
        self.stp = torch.from_numpy(stp.view(np.int32)).cuda()
        self.layout = hs.layout_of(page, rb, L, C, pool_rows, host_rows, ps, hs_)
        # the early fill's work counters (zeroed once; every call leaves them zero)
        self.sync = (torch.zeros(hs.HS_FILL_SYNC_WORDS, dtype=torch.int32, device="cuda")
                     if fill_sync else None)
        self.batch = hs.batch_of(bt.shape[0], bt.shape[1], self.pool_flat, self.host_pool, self.bt,
                                 self.hbt, self.ctx, self.hot, self.tok, self.stp, self.sync)

    def resolve(self, topk: np.ndarray, stamp: int, gather=True, pairs=None, mode="call"):
        R, L = topk.shape[:2]
        P, K = (1, topk.shape[2]) if topk.ndim == 3 else topk.shape[2:]
        t = torch.from_numpy(np.ascontiguousarray(topk)).cuda()
        rows = torch.empty(topk.shape, dtype=torch.int32, device="cuda")
        stats = torch.empty((R, L, 8), dtype=torch.int32, device="cuda")
        out = (torch.empty(topk.shape + (self.rb,), dtype=torch.uint8, device="cuda")
               if gather else None)
        pr = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).cuda() \
            if pairs is not None else None
        stages.run(mode, self.layout, self.batch, t, P, K, stamp, rows, out, stats, pr,
                   0 if pairs is None else len(pairs))
        torch.cuda.synchronize()
        return (rows.cpu().numpy(), stats.cpu().numpy(),
                None if out is None else out.cpu().numpy())

    def state(self):
        if self.pad:
            L = self.L
            for flat in (self.pool_flat.cpu(), self.host_flat):
                gaps = flat.view(L, -1)[:, -self.pad:]
                assert bool((gaps == 0xA5).all()), "bytes past a layer's rows were written"
        return (self.tok.cpu().numpy(), self.stp.cpu().numpy().view(np.uint32),
                self.pool.cpu().numpy(), self.host.numpy().copy())

    def close(self):
        self.host = None
        self.host_flat = None
        self.host_pool.close()


def _compare(case, inst_or_arrays, topk, stamp, pairs=None, page=None, mode="call"):
    a = inst_or_arrays
    g_rows, g_stats, g_out = case.resolve(topk, stamp, pairs=pairs, mode=mode)
    o_rows, o_stats, o_out = oracle.resolve(a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"],
                                            a["hot"], a["tok"], a["stp"],
                                            np.ascontiguousarray(topk), stamp, True,
                                            page=case.page)
    if pairs is not None and len(pairs):
        oracle.offload(a["pool"], a["host"], np.asarray(pairs, np.int32), page=case.page)
    tok, stp, pool, host = case.state()
    assert np.array_equal(g_rows, o_rows)
    assert np.array_equal(g_stats, o_stats)
    if mode != "in_place":           # there the output is only staging
        assert np.array_equal(g_out, o_out)
    assert np.array_equal(tok, a["tok"])
    assert np.array_equal(stp, a["stp"])
    assert np.array_equal(pool, a["pool"])
    assert np.array_equal(host, a["host"])
    return o_rows, o_stats


def _case_from_tiny(inst):
    return GpuCase(inst["page"], inst["pool"], inst["host"], inst["bt"], inst["hbt"],
                   inst["ctx"], inst["hot"], inst["tok"].copy(), inst["stp"].copy(),
                   inst["tok"].shape[2])


@pytest.mark.parametrize("mode", stages.MODES)
def test_worked_example_on_gpu(mode):
    inst = tiny_instance()
    case = _case_from_tiny(inst)
    try:
        lists = [[21, 5, 13, 2, 17, 9], [9, 1, 22, 13, 6, 14]]
        rows, _ = _compare(case, inst, np.array([[lists[0]]], np.int32), 1, mode=mode)
        assert rows.ravel().tolist() == [9, 37, 39, 36, 29, 38]
        rows, _ = _compare(case, inst, np.array([[lists[1]]], np.int32), 2, mode=mode)
        assert rows.ravel().tolist() == [38, 24, 10, 39, 25, 26]
        inst["bt"][0, 4] = -1
        case.bt[0, 4] = -1
        rows, _ = _compare(case, inst, np.array([[[17, 2, 10, 6, 20, 3]]], np.int32), 3,
                           mode=mode)
        assert rows.ravel().tolist() == [38, 36, 37, 25, 8, 27]
        rows, stats = _compare(case, inst, np.array([[[17, 2, 10, 6, 20, 3]]], np.int32), 4,
                               mode=mode)
        assert stats.ravel()[:3].tolist() == [1, 5, 0]
    finally:
        case.close()


@pytest.mark.parametrize("mode", stages.MODES)
def test_worked_example_plan_and_overflow_on_gpu(mode):
    inst = tiny_instance(C=4, hot_blocks=(9,))
    case = _case_from_tiny(inst)
    try:
        _compare(case, inst, np.array([[[21, 5, 13, 2, 17, 9]]], np.int32), 1, mode=mode)
        rows, stats = _compare(case, inst, np.array([[[[9, 1, 22], [13, 6, 14]]]], np.int32), 2,
                               mode=mode)
        assert rows.tolist() == [[[[38, 36, 10], [39, 37, -2]]]]
        assert stats.ravel().tolist() == [1, 2, 2, 1, 0, 0, 0, 0]
    finally:
        case.close()


def random_arrays(rs: np.random.Generator, R, L, C, page, rb, n_pages, n_blocks, n_host,
                  hostile=False):
    """A random batch.  Hot blocks of different requests are disjoint (a
    caller precondition); with ``hostile`` the tables also point outside the
    pools, some hot blocks are unusable, stamps are non-monotone and some
    slots hold stale tokens past the tables' span."""
    pool = rs.integers(0, 256, size=(L, n_blocks * page, rb), dtype=np.uint8)
    host = rs.integers(0, 256, size=(L, n_host * page, rb), dtype=np.uint8)
    hb_per = C // page
    perm = rs.permutation(n_blocks)
    hot = perm[:R * hb_per].reshape(R, hb_per).astype(np.int32)
    rest = perm[R * hb_per:]
    bt = np.where(rs.random((R, n_pages)) < 0.5, -1,
                  rs.choice(rest, size=(R, n_pages))).astype(np.int32)
    hbt = np.where(rs.random((R, n_pages)) < 0.1, -1,
                   rs.integers(0, n_host, size=(R, n_pages))).astype(np.int32)
    ctx = rs.integers(page, n_pages * page + 1, size=R).astype(np.int32)
    if hostile:
        bt[rs.random((R, n_pages)) < 0.05] = n_blocks + 3
        bt[rs.random((R, n_pages)) < 0.05] = -7
        hbt[rs.random((R, n_pages)) < 0.05] = n_host + 1
        hot[rs.random(hot.shape) < 0.1] = n_blocks + 5
        ctx[0] = n_pages * page + 50  # context longer than the table
    tok = np.full((R, L, C), -1, np.int32)
    stp = np.zeros((R, L, C), np.uint32)
    for r in range(R):
        for layer in range(L):
            k = rs.integers(0, C + 1)
            q = rs.choice(C, size=k, replace=False)
            tok[r, layer, q] = rs.choice(n_pages * page, size=k, replace=False)
            stp[r, layer, q] = rs.integers(1, 9, size=k)
            if hostile:
                stp[r, layer, rs.choice(C, size=C // 8, replace=False)] = \
                    rs.integers(1, 1 << 32, size=C // 8, dtype=np.uint64).astype(np.uint32)
                # stale tokens no list can hold: past the tables' span (the
                # fill's slot bitmap covers the span only) and far past it
                g = rs.choice(C, size=max(1, C // 64), replace=False)
                tok[r, layer, g] = n_pages * page + rs.choice(4 * C, size=g.size, replace=False)
                tok[r, layer, g[0]] = (1 << 30) + layer
    return dict(pool=pool, host=host, bt=bt, hbt=hbt, ctx=ctx, hot=hot, tok=tok, stp=stp)


def random_lists(rs, R, L, P, K, ctx, dup=0.1, pad=0.05, bad=0.03):
    out = np.empty((R, L, P, K), np.int32)
    for r in range(R):
        c = int(ctx[r])
        for layer in range(L):
            for p in range(P):
                v = rs.integers(0, c, size=K)
                d = rs.random(K) < dup
                v[d] = rs.choice(v, size=int(d.sum()))
                v[rs.random(K) < pad] = -1
                b = rs.random(K) < bad
                v[b] = rs.choice([-5, c, c + 7, 1 << 30], size=int(b.sum()))
                out[r, layer, p] = v
    return out


CASES = [
    # name, R, L, P, K, C, page, rb, n_pages, hostile
    ("ragged_k", 3, 2, 1, 1000, 2048, 64, 656, 200, False),
    ("k1", 4, 1, 1, 1, 64, 64, 656, 30, False),
    ("max_entries", 2, 1, 4, 2048, 8192, 64, 656, 400, False),
    ("max_capacity", 2, 1, 1, 2048, 8192, 64, 656, 300, False),
    # speculative decoding's sizing: (3 speculative tokens + 2) x 2048 slots for
    # a 4-position plan, and the largest capacity the resolver takes
    ("mtp_capacity", 2, 1, 4, 2048, 10240, 64, 656, 400, False),
    ("max_capacity_12k", 2, 1, 1, 2048, 12288, 64, 656, 400, False),
    # the resolver's largest LDS plan: 4 x 2048 entries with 12,288 slots
    ("max_plan_12k", 2, 1, 4, 2048, 12288, 64, 656, 500, False),
    ("max_plan_12k_hostile", 2, 1, 4, 2048, 12288, 64, 656, 500, True),
    ("hostile_c9216", 3, 1, 2, 900, 9216, 64, 656, 300, True),
    ("min_capacity", 5, 1, 1, 300, 64, 64, 656, 40, False),
    ("page16", 3, 2, 2, 700, 1024, 16, 656, 900, False),
    ("page128_rb64", 3, 1, 1, 1500, 2048, 128, 64, 80, False),
    ("rb1024", 2, 3, 1, 513, 512, 64, 1024, 50, False),
    # rows of one 16-byte piece (the fill's piece division has no multiplier)
    ("rb16", 4, 2, 2, 431, 352, 32, 16, 193, True),
    # the largest rows the resolving calls take (256 pieces), at the most
    # entries a request-layer holds (the fill's piece counters at their largest)
    ("rb4096", 2, 1, 2, 500, 256, 16, 4096, 20, True),
    ("rb4096_max_entries", 1, 1, 4, 2048, 4096, 64, 4096, 80, False),
    # pages of one token and of 1024 and 4096 tokens
    ("page1", 3, 1, 1, 200, 64, 1, 656, 400, False),
    ("page1024", 3, 1, 1, 700, 2048, 1024, 16, 12, False),
    ("page4096_hostile", 2, 2, 2, 500, 4096, 4096, 48, 5, True),
    ("hostile", 4, 2, 3, 600, 2048, 64, 656, 100, True),
    ("hostile_small", 6, 1, 1, 37, 128, 32, 656, 12, True),
    # more request-layers than CUs: the fused launch interleaves its resolver
    # and gather workgroups (260 is not a multiple of their groups of 8)
    ("many_request_layers", 130, 2, 1, 300, 512, 64, 656, 40, False),
]


@pytest.mark.parametrize("mode", stages.MODES)
@pytest.mark.parametrize("name,R,L,P,K,C,page,rb,n_pages,hostile", CASES,
                         ids=[c[0] for c in CASES])
def test_random_cases(name, R, L, P, K, C, page, rb, n_pages, hostile, mode):
    rs = np.random.default_rng(zlib.crc32(name.encode()))
    n_blocks = R * (C // page) + n_pages * R // 2 + 8
    a = random_arrays(rs, R, L, C, page, rb, n_pages, n_blocks, n_pages, hostile)
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C)
    try:
        for step in range(4):
            _say(f"[edges] {name} {mode} step {step}")
            lists = random_lists(rs, R, L, P, K, a["ctx"])
            topk = lists[:, :, 0] if P == 1 else lists
            pairs = None
            if step == 2:
                n = 5
                pairs = np.stack([rs.integers(0, n_blocks, n), rs.choice(n_pages, n, replace=False)], 1)
                if hostile:
                    pairs[0, 0] = n_blocks + 1
                    pairs[1, 1] = -2
            _compare(case, a, topk, 10 + 3 * step - (step == 3) * 7, pairs=pairs, mode=mode)
    finally:
        case.close()


def _sweep_shape(seed):
    """Shape of sweep case ``seed``: page, capacity, batch, positions, list
    length and row size drawn from the seed, the pools kept under ~48 MB."""
    rs = np.random.default_rng(1000 + seed)
    page = int(rs.choice([16, 32, 64, 128]))
    C = page * int(rs.integers(1, 4096 // page + 1))
    R = int(rs.integers(1, 13))
    L = int(rs.integers(1, 4))
    P = int(rs.choice([1, 1, 2, 3, 4]))
    K = int(rs.integers(1, min(1500, 8192 // P) + 1))
    rb = int(rs.choice([656, 656, 16, 48, 1024]))
    n_pages = max(int(rs.integers(4, 301)), C // page + 1)  # slot tokens come from the span
    while R > 1 and L * (R * (C // page) + n_pages * R // 2 + 8 + n_pages) * page * rb > 48 << 20:
        R -= 1
    return rs, R, L, P, K, C, page, rb, n_pages, bool(seed % 2)


SWEEP = list(range(48))


@pytest.mark.parametrize("seed", SWEEP)
def test_random_shapes_sweep(seed):
    """Random shapes, one stage mode each (the modes in turn), three steps
    with an offload in the second, hostile tables on odd seeds, the early
    fill's work counters on half the seeds."""
    rs, R, L, P, K, C, page, rb, n_pages, hostile = _sweep_shape(seed)
    mode = stages.MODES[seed % len(stages.MODES)]
    n_blocks = R * (C // page) + n_pages * R // 2 + 8
    a = random_arrays(rs, R, L, C, page, rb, n_pages, n_blocks, n_pages, hostile)
    sync = seed % 4 >= 2
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C, fill_sync=sync)
    try:
        for step in range(3):
            _say(f"[edges] sweep {seed} R={R} L={L} P={P} K={K} C={C} page={page} rb={rb} "
                 f"pages={n_pages} hostile={hostile} fill_sync={sync} {mode} step {step}")
            lists = random_lists(rs, R, L, P, K, a["ctx"])
            topk = lists[:, :, 0] if P == 1 else lists
            pairs = None
            if step == 1:
                n = min(4, n_pages)
                pairs = np.stack([rs.integers(0, n_blocks, n),
                                  rs.choice(n_pages, n, replace=False)], 1)
            _compare(case, a, topk, 5 + 2 * step, pairs=pairs, mode=mode)
            if sync:
                assert int(torch.count_nonzero(case.sync)) == 0, "work counters left set"
    finally:
        case.close()


def _wide_shape(seed):
    """A launch of 130-400 request-layers with short lists: more workgroups
    than the chip holds at once (interleaved resolvers and gathers, miss
    workgroups taking many items), rows sized to keep the pools small."""
    rs = np.random.default_rng(9000 + seed)
    page = int(rs.choice([16, 64]))
    C = page * int(rs.integers(1, 1024 // page + 1))
    L = int(rs.integers(1, 4))
    R = int(rs.integers(130 // L + 1, 400 // L + 1))
    P = int(rs.choice([1, 2]))
    K = int(rs.integers(1, 301))
    n_pages = max(int(rs.integers(4, 40)), C // page + 1)
    rb = 656
    for cand in (656, 48, 16):
        rb = cand
        if L * (R * (C // page) + n_pages * R // 2 + 8 + n_pages) * page * rb <= 64 << 20:
            break
    return rs, R, L, P, K, C, page, rb, n_pages


@pytest.mark.parametrize("seed", list(range(10)))
def test_wide_launch_sweep(seed):
    """Random wide launches in every stage mode (the modes in turn), half with
    the fill's work counters, three steps with an offload in the second."""
    rs, R, L, P, K, C, page, rb, n_pages = _wide_shape(seed)
    mode = stages.MODES[seed % len(stages.MODES)]
    n_blocks = R * (C // page) + n_pages * R // 2 + 8
    a = random_arrays(rs, R, L, C, page, rb, n_pages, n_blocks, n_pages, seed % 3 == 2)
    sync = seed % 2 == 1
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C, fill_sync=sync)
    try:
        for step in range(3):
            _say(f"[edges] wide {seed} R={R} L={L} P={P} K={K} C={C} page={page} rb={rb} "
                 f"fill_sync={sync} {mode} step {step}")
            lists = random_lists(rs, R, L, P, K, a["ctx"])
            topk = lists[:, :, 0] if P == 1 else lists
            pairs = None
            if step == 1:
                n = min(4, n_pages)
                pairs = np.stack([rs.integers(0, n_blocks, n),
                                  rs.choice(n_pages, n, replace=False)], 1)
            _compare(case, a, topk, 5 + 2 * step, pairs=pairs, mode=mode)
            if sync:
                assert int(torch.count_nonzero(case.sync)) == 0, "work counters left set"
    finally:
        case.close()


@pytest.mark.parametrize("mode", stages.MODES)
def test_padded_layer_strides(mode):
    """Both pools with layer strides past their rows (4,112 bytes of
    untouchable bytes after every layer): rows, stats, gathered bytes, state
    and both pools as the oracle's, and the gaps unwritten, through every
    path, offload included."""
    rs = np.random.default_rng(zlib.crc32(f"padded-{mode}".encode()))
    R, L, P, K, C, page, rb, n_pages = 3, 3, 2, 300, 512, 32, 656, 40
    n_blocks = R * (C // page) + n_pages * R // 2 + 8
    a = random_arrays(rs, R, L, C, page, rb, n_pages, n_blocks, n_pages, True)
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C, pad=4112)
    try:
        for step in range(3):
            _say(f"[edges] padded strides {mode} step {step}")
            topk = random_lists(rs, R, L, P, K, a["ctx"])
            pairs = None
            if step == 1:
                pairs = np.stack([rs.integers(0, n_blocks, 4), rs.choice(n_pages, 4, replace=False)], 1)
            _compare(case, a, topk, 5 + 2 * step, pairs=pairs, mode=mode)
    finally:
        case.close()


def test_empty_batch_and_zero_pairs():
    import serving_memory_tier_amd as hs
    a = random_arrays(np.random.default_rng(1), 1, 1, 64, 64, 656, 4, 8, 4)
    case = GpuCase(64, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), 64)
    try:
        empty = hs.batch_of(0, 4, case.pool, case.host_pool, case.bt, case.hbt, case.ctx,
                            case.hot, case.tok, case.stp)
        t = torch.zeros((8,), dtype=torch.int32, device="cuda")
        hs.hs_resolve(case.layout, empty, t, 16, 1, t, None, t)
        hs.hs_offload_prefix_pages(case.layout, case.pool, case.host_pool, t, 0)
        hs.hs_gather(case.layout, case.pool, t, 0, 16, t)
        torch.cuda.synchronize()
    finally:
        case.close()


@pytest.mark.parametrize("rb", [656, 64, 1024, 16, 48])
def test_gather_entry_point(rb):
    import serving_memory_tier_amd as hs
    rs = np.random.default_rng(rb)
    L, rows_per_layer = 3, 64 * 50
    pool = rs.integers(0, 256, size=(L, rows_per_layer, rb), dtype=np.uint8)
    rows = rs.integers(-4, rows_per_layer + 9, size=(5, L, 1333)).astype(np.int32)
    rows[0, 0, :7] = [-1, -2, -3, rows_per_layer, rows_per_layer - 1, 0, 2 ** 31 - 1]
    lay = hs.layout_of(64, rb, L, 64, rows_per_layer, 0)
    gp = torch.from_numpy(pool).cuda()
    gr = torch.from_numpy(rows).cuda()
    out = torch.empty((5, L, 1333, rb), dtype=torch.uint8, device="cuda")
    hs.hs_gather(lay, gp, gr, 5, 1333, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.gather(pool, rows))


@pytest.mark.parametrize("page,rb", [(64, 656), (16, 16), (128, 48), (32, 1024)])
def test_offload_entry_point(page, rb):
    import serving_memory_tier_amd as hs
    rs = np.random.default_rng(9 + page + rb)
    L, nb, nh = 4, 40, 30
    pool = rs.integers(0, 256, size=(L, nb * page, rb), dtype=np.uint8)
    host = rs.integers(0, 256, size=(L, nh * page, rb), dtype=np.uint8)
    pairs = np.stack([rs.integers(0, nb, 12), rs.choice(nh, 12, replace=False)], 1).astype(np.int32)
    pairs[3] = [nb, 2]
    pairs[4] = [1, -1]
    lay = hs.layout_of(page, rb, L, page, nb * page, nh * page)
    gp = torch.from_numpy(pool).cuda()
    hp = hs.HostPool(host.size)
    try:
        hv = hp.tensor.view(host.shape)
        hv.copy_(torch.from_numpy(host))
        hs.hs_offload_prefix_pages(lay, gp, hp, torch.from_numpy(pairs).cuda(), 12)
        torch.cuda.synchronize()
        oracle.offload(pool, host, pairs, page=page)
        assert np.array_equal(hv.numpy(), host)
        assert np.array_equal(gp.cpu().numpy(), pool)
    finally:
        hv = None
        hp.close()


GROUPED = [
    # name, R, L, G, P, K, C, page, rb, n_pages, hostile
    ("g2_l4", 3, 4, 2, 1, 700, 1024, 64, 656, 120, False),
    ("g4_l4_plan", 2, 4, 4, 2, 512, 2048, 64, 656, 150, False),
    ("g2_hostile", 4, 4, 2, 1, 300, 512, 32, 656, 40, True),
    ("g3_l6_rb64", 2, 6, 3, 1, 400, 512, 16, 64, 60, False),
]


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "copies_only"])
@pytest.mark.parametrize("name,R,L,G,P,K,C,page,rb,n_pages,hostile", GROUPED,
                         ids=[c[0] for c in GROUPED])
def test_random_grouped_cases(name, R, L, G, P, K, C, page, rb, n_pages, hostile, gather):
    """hs_resolve_grouped against the oracle's grouped resolve: state and lists
    per layer group, copies and gathered rows per layer."""
    rs = np.random.default_rng(zlib.crc32(name.encode()))
    _run_grouped(rs, R, L, G, P, K, C, page, rb, n_pages, hostile, gather, name)


def _run_grouped(rs, R, L, G, P, K, C, page, rb, n_pages, hostile, gather, label):
    import serving_memory_tier_amd as hs
    n_blocks = R * (C // page) + n_pages * R // 2 + 8
    a = random_arrays(rs, R, L, C, page, rb, n_pages, n_blocks, n_pages, hostile)
    NG = L // G
    a["tok"] = np.ascontiguousarray(a["tok"][:, :NG])
    a["stp"] = np.ascontiguousarray(a["stp"][:, :NG])
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C)
    try:
        for step in range(3):
            _say(f"[edges] grouped {label} gather={gather} step {step}")
            lists = random_lists(rs, R, NG, P, K, a["ctx"])
            topk = np.ascontiguousarray(lists[:, :, 0] if P == 1 else lists)
            stamp = 5 + 2 * step
            t = torch.from_numpy(topk).cuda()
            rows = torch.empty(topk.shape, dtype=torch.int32, device="cuda")
            stats = torch.empty((R, NG, 8), dtype=torch.int32, device="cuda")
            out = (torch.empty((R, L) + topk.shape[2:] + (rb,), dtype=torch.uint8, device="cuda")
                   if gather else None)
            hs.hs_resolve_grouped(case.layout, case.batch, G, t, P, K, stamp, rows, out, stats)
            torch.cuda.synchronize()
            o_rows, o_stats, o_out = oracle.resolve_grouped(
                a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"], a["tok"], a["stp"],
                topk, stamp, G, gather, page=page)
            tok, stp, pool, host = case.state()
            assert np.array_equal(rows.cpu().numpy(), o_rows)
            assert np.array_equal(stats.cpu().numpy(), o_stats)
            if gather:
                assert np.array_equal(out.cpu().numpy(), o_out)
            assert np.array_equal(tok, a["tok"])
            assert np.array_equal(stp, a["stp"])
            assert np.array_equal(pool, a["pool"])
    finally:
        case.close()


def _grouped_sweep_shape(seed):
    """Shape of grouped sweep case ``seed``, the pools kept under ~48 MB."""
    rs = np.random.default_rng(5000 + seed)
    page = int(rs.choice([16, 32, 64]))
    C = page * int(rs.integers(1, 2048 // page + 1))
    G = int(rs.integers(2, 5))
    L = G * int(rs.integers(1, 4))
    R = int(rs.integers(1, 9))
    P = int(rs.choice([1, 1, 2]))
    K = int(rs.integers(1, 1001))
    rb = int(rs.choice([656, 656, 16, 48, 1024]))
    n_pages = max(int(rs.integers(4, 201)), C // page + 1)  # slot tokens come from the span
    while R > 1 and L * (R * (C // page) + n_pages * R // 2 + 8 + n_pages) * page * rb > 48 << 20:
        R -= 1
    return rs, R, L, G, P, K, C, page, rb, n_pages, bool(seed % 2), seed % 3 != 0


GROUPED_SWEEP = list(range(24))


@pytest.mark.parametrize("seed", GROUPED_SWEEP)
def test_random_grouped_sweep(seed):
    """Random shapes for hs_resolve_grouped (groups of 2-4 layers, 1-3 groups,
    rows of 16 to 1024 bytes), with and without the gathered output."""
    rs, R, L, G, P, K, C, page, rb, n_pages, hostile, gather = _grouped_sweep_shape(seed)
    _run_grouped(rs, R, L, G, P, K, C, page, rb, n_pages, hostile, gather,
                 f"sweep {seed} R={R} L={L} G={G} P={P} K={K} C={C} page={page} rb={rb}")


@pytest.mark.parametrize("mode", stages.MODES)
@pytest.mark.parametrize("C", [512, 10240])
def test_victims_across_many_stamp_groups(C, mode):
    """Every slot holds a token the lists do not ask for, each slot with a
    stamp of its own, and a list misses more tokens than sixteen stamp groups
    hold: the resolver takes its victims through its full sort of the
    candidates by stamp instead of group by group."""
    rs = np.random.default_rng(zlib.crc32(f"groups{C}".encode()))
    page, rb, R, L = 64, 656, 2, 1
    K = min(2048, C // 2)
    n_pages = 2 * (C // page) + 4 * (K // page)
    ctx = np.full(R, n_pages * page, np.int32)
    n_blocks = R * (C // page) + 4
    pool = rs.integers(0, 256, size=(L, n_blocks * page, rb), dtype=np.uint8)
    host = rs.integers(0, 256, size=(L, R * n_pages * page, rb), dtype=np.uint8)
    bt = np.full((R, n_pages), -1, np.int32)                    # nothing resident
    hbt = np.stack([rs.permutation(n_pages) + r * n_pages for r in range(R)]).astype(np.int32)
    hot = (np.arange(R * (C // page)).reshape(R, C // page) + 2).astype(np.int32)
    tok = np.stack([rs.permutation(C) for _ in range(R)]).reshape(R, L, C).astype(np.int32)
    stp = np.stack([rs.permutation(C) + 1 for _ in range(R)]).reshape(R, L, C).astype(np.uint32)
    a = dict(pool=pool, host=host, bt=bt, hbt=hbt, ctx=ctx, hot=hot, tok=tok, stp=stp)
    case = GpuCase(page, pool, host, bt, hbt, ctx, hot, tok.copy(), stp.copy(), C)
    try:
        # step 1: K distinct misses beyond the slots' tokens; step 2: half of
        # them again (now hits) and fresh misses
        first = np.stack([rs.choice(np.arange(C, n_pages * page), K, replace=False)
                          for _ in range(R)]).reshape(R, L, K).astype(np.int32)
        _say(f"[edges] stamp groups C={C} {mode} step 1")
        _, st = _compare(case, a, first, C + 5, mode=mode)
        assert (st[..., 2] == K).all() and (st[..., 3] == 0).all()
        second = first.copy()
        for r in range(R):
            fresh = np.setdiff1d(np.arange(C, n_pages * page), first[r, 0])
            second[r, 0, K // 2:] = rs.choice(fresh, K - K // 2, replace=False)
        _say(f"[edges] stamp groups C={C} {mode} step 2")
        _, st = _compare(case, a, second, C + 9, mode=mode)
        assert (st[..., 1] == K // 2).all()
    finally:
        case.close()


def _max_stamp_instance(rs, R, L, C, page, n_pages, n_resident):
    """Slots 0..page-1 sit in an unusable hot block (outside the pool) and hold
    stamp 5; slots page..2*page-1 hold tokens the lists will ask for (hits)
    at stamp 7; every other slot holds a token nobody asks for at the largest
    stamp, 0xffffffff.  Pages below n_pages - n_resident are host-only."""
    rb = 656
    n_blocks = R * (C // page) + R * n_resident + 4
    pool = rs.integers(0, 256, size=(L, n_blocks * page, rb), dtype=np.uint8)
    host = rs.integers(0, 256, size=(L, R * n_pages * page, rb), dtype=np.uint8)
    perm = rs.permutation(n_blocks)
    hot = perm[:R * (C // page)].reshape(R, C // page).astype(np.int32)
    hot[:, 0] = n_blocks + 5                                    # unusable
    rest = perm[R * (C // page):]
    bt = np.full((R, n_pages), -1, np.int32)
    bt[:, n_pages - n_resident:] = rest[:R * n_resident].reshape(R, n_resident)
    hbt = np.stack([rs.permutation(n_pages) + r * n_pages for r in range(R)]).astype(np.int32)
    ctx = np.full(R, n_pages * page, np.int32)
    n_nonres = (n_pages - n_resident) * page
    tok = np.empty((R, L, C), np.int32)
    stp = np.full((R, L, C), 0xFFFFFFFF, np.uint32)
    stp[:, :, :page] = 5
    stp[:, :, page:2 * page] = 7
    order = np.empty((R, L, n_nonres), np.int64)
    for r in range(R):
        for layer in range(L):
            order[r, layer] = rs.permutation(n_nonres)
            tok[r, layer] = order[r, layer, :C]
    return dict(pool=pool, host=host, bt=bt, hbt=hbt, ctx=ctx, hot=hot, tok=tok, stp=stp), order


@pytest.mark.parametrize("mode", stages.MODES)
@pytest.mark.parametrize("more_misses", [False, True], ids=["fewer_misses", "more_misses"])
def test_victims_at_the_largest_stamp(more_misses, mode):
    """The LRU slot of "How it works" is chosen among usable non-hit slots
    only, whatever their stamps: here every candidate holds the largest
    stamp, 0xffffffff, while hit slots and an unusable hot block sit at the
    lowest slot indices.  With fewer misses than candidates every miss gets a
    slot; with more, the extra misses overflow.  A second call, itself at
    stamp 0xffffffff, evicts the first call's victims before the rest."""
    rs = np.random.default_rng(zlib.crc32(f"maxstamp{more_misses}".encode()))
    page, R, L, C = 64, 2, 2, 512
    n_pages, n_resident = 40, 10
    a, order = _max_stamp_instance(rs, R, L, C, page, n_pages, n_resident)
    case = GpuCase(page, a["pool"], a["host"], a["bt"], a["hbt"], a["ctx"], a["hot"],
                   a["tok"].copy(), a["stp"].copy(), C)
    n_fresh = 400 if more_misses else 100
    P, K = (2, 256) if more_misses else (1, 256)
    res0 = (n_pages - n_resident) * page
    try:
        for step, stamp in enumerate((9, 0xFFFFFFFF)):
            lists = np.empty((R, L, P * K), np.int32)
            for r in range(R):
                for layer in range(L):
                    o = order[r, layer]
                    hits = o[page:2 * page]                        # hit slots' tokens
                    unusable = o[:20]                              # held by unusable slots: misses
                    fresh = o[C + step * n_fresh:C + (step + 1) * n_fresh]
                    n_res = P * K - hits.size - unusable.size - fresh.size
                    resident = rs.integers(res0, n_pages * page, size=n_res)
                    v = np.concatenate([hits, unusable, fresh, resident])
                    lists[r, layer] = rs.permutation(v)
            topk = lists if P == 1 else lists.reshape(R, L, P, K)
            _say(f"[edges] largest stamp more_misses={more_misses} {mode} step {step}")
            _, st = _compare(case, a, np.ascontiguousarray(topk), stamp, mode=mode)
            if step == 0:
                assert (st[..., 1] == page).all()                 # every hit slot hit
                m = 20 + n_fresh
                cand = C - 2 * page
                assert (st[..., 2] == min(m, cand)).all()
                assert (st[..., 3] == max(0, m - cand)).all()
                # no hit slot and no unusable slot was taken
                assert (a["stp"][:, :, :page] == 5).all()
                assert (a["stp"][:, :, page:2 * page] == 9).all()
    finally:
        case.close()


@pytest.mark.parametrize("mode", stages.MODES)
def test_overflow_at_size(mode):
    """A 4-position plan of 2048 entries per position over a host-only context:
    more distinct misses than the 4096 slots hold, so the largest ones
    overflow (row -2, nothing copied for them), at the workload size."""
    rs = np.random.default_rng(zlib.crc32(b"overflow_at_size"))
    page, rb, R, L, P, K, C = 64, 656, 4, 1, 4, 2048, 4096
    n_pages = 400
    n_blocks = R * (C // page) + 4
    pool = rs.integers(0, 256, size=(L, n_blocks * page, rb), dtype=np.uint8)
    host = rs.integers(0, 256, size=(L, R * n_pages * page, rb), dtype=np.uint8)
    hot = rs.permutation(n_blocks)[:R * (C // page)].reshape(R, C // page).astype(np.int32)
    bt = np.full((R, n_pages), -1, np.int32)                     # nothing resident
    hbt = np.stack([rs.permutation(n_pages) + r * n_pages for r in range(R)]).astype(np.int32)
    ctx = np.full(R, n_pages * page, np.int32)
    tok = np.full((R, L, C), -1, np.int32)
    stp = np.zeros((R, L, C), np.uint32)
    a = dict(pool=pool, host=host, bt=bt, hbt=hbt, ctx=ctx, hot=hot, tok=tok, stp=stp)
    case = GpuCase(page, pool, host, bt, hbt, ctx, hot, tok.copy(), stp.copy(), C)
    try:
        prev = None
        for step in range(3):
            lists = rs.integers(0, n_pages * page, size=(R, L, P, K)).astype(np.int32)
            if prev is not None:     # half of the first position repeats the last step's
                lists[:, :, 0, :K // 2] = prev[:, :, 0, :K // 2]
            prev = lists
            _say(f"[edges] overflow at size {mode} step {step}")
            _, st = _compare(case, a, lists, 3 + step, mode=mode)
            assert (st[..., 3] > 1000).all()
            assert (st.sum(axis=-1) == P * K).all()
    finally:
        case.close()
