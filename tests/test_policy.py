"""The host-side residency policy (libhs_policy.so) against the rules the pages
give it, on the CPU: GPU-first (nothing leaves the pool while it has room),
the tail never leaves, a page becomes a null placeholder only after its host
copy was queued in an earlier step, the coldest eligible pages go first, a
request holds a hot lease exactly while it has a placeholder, pool blocks are
never used twice, and the edits reproduce the policy's own tables."""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import serving_memory_tier_amd as hs
from serving_memory_tier_amd import policy as pol


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(pol.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build_policy()
    pol.lib()


class Mirror:
    """The caller's view: tables and leases rebuilt from the edits alone."""

    def __init__(self, R, max_pages, hb):
        self.bt = np.full((R, max_pages), -1, np.int32)
        self.hbt = np.full((R, max_pages), -1, np.int32)
        self.hot = np.full((R, hb), -1, np.int32)
        self.queued = {}    # (r, page) -> call index the host copy was queued in

    def apply(self, e: pol.Edits, call: int, page_of_block):
        for r, p, v in e.bt_set:
            self.bt[r, p] = v
        for r, p, v in e.hbt_set:
            self.hbt[r, p] = v
        for r, j, v in e.hot_set:
            self.hot[r, j] = v
        for db, hb in e.offload:
            self.queued[page_of_block[int(db)]] = call


def _pages(ctx, page):
    return (ctx + page - 1) // page


def _simulate(seed, R=6, page=16, n_blocks=60, hb=2, tail=2, steps=120, K=24, admit_host=True):
    rs = np.random.default_rng(seed)
    max_pages = 64
    p = pol.Policy(page, n_blocks, 4096, R, max_pages, hb, tail)
    m = Mirror(R, max_pages, hb)
    last_use = np.zeros((R, max_pages), np.int64)
    ctx = rs.integers(3 * page, 12 * page, size=R)
    call = 0
    stats = dict(evicted=0, leased=0)

    def page_of_block():
        out = {}
        for r in range(R):
            for pg in range(max_pages):
                if m.bt[r, pg] >= 0:
                    out[int(m.bt[r, pg])] = (r, pg)
        return out

    for r in range(R):
        host = None
        if admit_host and r % 2:
            # a reused prefix: complete pages already on host (private host ids 3000+)
            host = np.array([3000 + 64 * r + q for q in range(int(ctx[r]) // page)], np.int32)
        e = p.admit(r, int(ctx[r]), host)
        call += 1
        m.apply(e, call, page_of_block())
    prev = None
    for s in range(1, steps + 1):
        free_before = p.free_blocks()
        new_ctx = ctx + rs.integers(0, 6, size=R)
        topk = None
        if prev is not None:
            topk = prev
            for r in range(R):
                for t in prev[r]:
                    if 0 <= t < ctx[r]:
                        last_use[r, t // page] = s
        tails_before = {r: _pages(int(new_ctx[r]), page) for r in range(R)}
        e = p.step(s, np.arange(R), new_ctx, topk)
        call += 1
        bt_before = m.bt.copy()
        m.apply(e, call, page_of_block())
        ctx = new_ctx
        stats["evicted"] += e.evicted
        stats["leased"] += e.leased

        # the edits reproduce the policy's own tables
        for r in range(R):
            bt, hbt, hot = p.tables(r)
            assert np.array_equal(bt, m.bt[r]) and np.array_equal(hbt, m.hbt[r])
            assert np.array_equal(hot, m.hot[r])
        # pool blocks: resident pages and leases are disjoint and account for the pool
        used = [int(b) for b in m.bt.ravel() if b >= 0] + [int(b) for b in m.hot.ravel() if b >= 0]
        assert len(used) == len(set(used))
        assert all(0 <= b < n_blocks for b in used)
        assert len(used) + p.free_blocks() == n_blocks
        # GPU-first: evictions only when the step's demand exceeded the free blocks
        nulled = [(int(r), int(pg)) for r, pg, v in e.bt_set if v < 0 and bt_before[r, pg] >= 0]
        assert len(nulled) == e.evicted
        if nulled:
            new_blocks = sum(1 for r, pg, v in e.bt_set if v >= 0)
            assert free_before < new_blocks + e.leased * hb
        for r, pg in nulled:
            # not the tail, complete, and its host copy queued in an earlier call
            assert pg < tails_before[r] - tail
            assert (pg + 1) * page <= ctx[r]
            assert m.hbt[r, pg] >= 0 or m.queued.get((r, pg), call) < call
        # coldest first: no page left resident and eligible is colder than an evicted one
        if nulled:
            worst = max((last_use[r, pg], r, pg) for r, pg in nulled)
            for r in range(R):
                for pg in range(_pages(int(ctx[r]), page) - tail):
                    if m.bt[r, pg] < 0 or (pg + 1) * page > ctx[r]:
                        continue
                    eligible = m.hbt[r, pg] >= 0 or m.queued.get((r, pg), call) < call
                    if eligible:
                        assert (last_use[r, pg], r, pg) > worst
        # the tail of every request is resident
        for r in range(R):
            np_ = _pages(int(ctx[r]), page)
            assert (m.bt[r, max(0, np_ - tail):np_] >= 0).all()
        # a lease exactly while a placeholder exists; resets for new leases
        for r in range(R):
            has_ph = bool((m.bt[r, :_pages(int(ctx[r]), page)] < 0).any())
            assert has_ph == bool((m.hot[r] >= 0).all())
            assert (m.hot[r] >= 0).all() or (m.hot[r] < 0).all()
        granted = {int(r) for r, j, v in e.hot_set if v >= 0}
        assert granted == set(e.reset.tolist())
        prev = [rs.integers(0, int(ctx[r]), size=K) for r in range(R)]
    # finishing returns everything
    for r in range(R):
        e = p.finish(r)
        m.apply(e, call + 1, {})
    assert p.free_blocks() == n_blocks
    p.close()
    return stats


@pytest.mark.parametrize("seed", range(6))
def test_policy_rules_under_pressure(seed):
    st = _simulate(seed)
    assert st["evicted"] > 0 and st["leased"] > 0   # the pool did run short


def test_no_pressure_no_eviction():
    st = _simulate(11, n_blocks=4000, admit_host=False)
    assert st["evicted"] == 0 and st["leased"] == 0


def test_admission_of_a_host_prefix_takes_a_lease():
    p = pol.Policy(16, 40, 100, 2, 32, 2, 2)
    e = p.admit(0, 16 * 10 + 5, np.arange(10, dtype=np.int32))
    bt, hbt, hot = p.tables(0)
    # pages 0..8 host-only (page 9 is in the tail with the partial page 10)
    assert (bt[:9] == -1).all() and (bt[9:11] >= 0).all()
    assert (hbt[:10] == np.arange(10)).all()
    assert (hot >= 0).all() and e.leased == 1 and e.reset.tolist() == [0]
    assert p.free_blocks() == 40 - 2 - 2
    p.close()


def test_pool_exhaustion_is_an_error():
    p = pol.Policy(16, 3, 100, 2, 32, 2, 1)
    p.admit(0, 16, None)                     # one page
    with pytest.raises(pol.PolicyError) as ei:
        p.step(1, [0], [16 * 5])             # four new pages, nothing evictable
    assert ei.value.status == pol.ERR_POOL_EXHAUSTED


def test_rejects_bad_arguments():
    with pytest.raises(pol.PolicyError):
        pol.Policy(0, 10, 10, 1, 4, 1, 1)
    p = pol.Policy(16, 10, 10, 2, 4, 1, 1)
    with pytest.raises(pol.PolicyError):
        p.admit(5, 16)                       # no such request slot
    with pytest.raises(pol.PolicyError):
        p.admit(0, 16 * 5)                   # more pages than the table has
    p.admit(0, 16)
    with pytest.raises(pol.PolicyError):
        p.admit(0, 16)                       # already admitted
    with pytest.raises(pol.PolicyError):
        p.step(1, [0], [8])                  # context shrinks
    with pytest.raises(pol.PolicyError):
        p.step(1, [1], [32])                 # not admitted
    e = pol._Edits()
    r, c = np.zeros(1, np.int32), np.full(1, 16, np.int32)
    assert pol.lib().hs_policy_step_pages(p.h, r.ctypes.data, c.ctypes.data, 1, None, 4,
                                          ctypes.byref(e)) == pol.ERR_INVALID_ARGUMENT
    assert pol.lib().hs_policy_step_pages(p.h, r.ctypes.data, c.ctypes.data, 1, None, -1,
                                          ctypes.byref(e)) == pol.ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        p.step_pages([0], [16], np.zeros((2, 4), np.uint32))   # one row per request
    with pytest.raises(pol.PolicyError):
        pol.Policy(48, 10, 10, 1, 4, 1, 1)   # pages of a power-of-two size only
    p.close()
    assert hs.lib  # the GPU library's binding is importable alongside


@pytest.mark.parametrize("group", [1, 2])
def test_policy_driven_oracle_run(group):
    """The policy's edits drive the oracle step by step (blocks reused for new
    pages and leases, leases granted mid-run with an emptied hot buffer, host
    copies backing every nulled page): every gathered row still holds its
    token's content, and the hot buffer never serves a stale row."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from harness import OracleRun, expected_content, policy_workload
    wl, dec = policy_workload(group=group, L=2 * group)
    assert dec.evicted > 0 and dec.leased > wl.R // 2   # some resident requests got leases
    ora = OracleRun(wl)
    totals = np.zeros(8, np.int64)
    for i, s in enumerate(wl.steps):
        ora.pre(s)
        for r in s.reset:
            assert (ora.tok[r] == -1).all()
        rows, stats, out = ora.resolve(s)
        totals += stats.sum(axis=(0, 1))
        assert np.array_equal(out, expected_content(wl, s.topk, rows)), f"step {i}"
        ora.post(s)
    assert totals[1] > 0 and totals[2] > 0 and totals[0] > 0
    # every host copy the tables know of (reused prefixes and the copies the
    # policy queued) holds its page's content, every layer
    import hs_gen
    o = np.arange(hs_gen.PAGE)
    for r in range(wl.R):
        for p in np.nonzero(ora.hbt[r] >= 0)[0]:
            rows = int(ora.hbt[r, p]) * hs_gen.PAGE + o
            for layer in range(wl.L):
                exp = hs_gen.content_np(np.full(o.size, layer), np.full(o.size, wl.src[r]),
                                        p * hs_gen.PAGE + o)
                assert np.array_equal(ora.host[layer, rows], exp), (r, p, layer)


class PageUseDecider:
    """The policy driven by per-page coldness stamps (hs_policy_step_pages),
    the table hs_page_touch keeps on the GPU, here written by the oracle's
    page_touch from the previous step's lists at that step's stamp."""

    def __init__(self, R, n_blocks, n_host_blocks, max_pages, C, tail_pages, touch):
        self.p = pol.Policy(64, n_blocks, n_host_blocks, R, max_pages, C // 64, tail_pages)
        self.use = np.zeros((R, max_pages), np.uint32)
        self.ctx = np.zeros(R, np.int32)
        self.touch = touch

    def admit(self, r, ctx, host_block_of_page, resident_prefix):
        self.ctx[r] = ctx
        return self.p.admit(r, ctx, host_block_of_page, resident_prefix)

    def step(self, stamp, reqs, ctx, topk):
        if topk is not None:
            self.touch(self.ctx, topk, stamp - 1, self.use)
        self.ctx = np.asarray(ctx, np.int32).copy()
        return self.p.step_pages(reqs, ctx, self.use[np.asarray(reqs)])


def _same_edits(a, b):
    for sa, sb in zip(a.steps, b.steps):
        for f in ("bt_set", "hbt_set", "hot_set", "reset", "offload", "new_pages"):
            assert np.array_equal(getattr(sa, f), getattr(sb, f)), (sa.stamp, f)
    assert len(a.steps) == len(b.steps)


@pytest.mark.parametrize("group", [1, 2])
def test_page_stamps_drive_the_same_decisions_as_lists(group):
    """Coldness from per-page stamps (one word per page) and from the lists
    themselves rank pages alike, so the policy makes the same edits."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    import hs_gen
    import oracle
    from harness import policy_workload
    wl, dec = policy_workload(group=group, L=2 * group)
    assert dec.evicted > 0
    # the same workload, its decider reading page stamps
    holder = {}

    class Capture(PageUseDecider):
        def __init__(self, *a):
            super().__init__(*a, touch=oracle.page_touch)
            holder["d"] = self

    R, mp = wl.R, int(max(wl.max_pages, 1))
    d = Capture(R, wl.n_blocks, dec.p.cfg.num_host_blocks, dec.p.cfg.max_pages, wl.C,
                dec.p.cfg.tail_pages)
    spec = hs_gen.Spec(name=wl.name, seed=wl.seed, R=R, L=wl.L, K=wl.K, C=wl.C,
                       steps=len(wl.steps), ctx0=wl.ctx0.astype(np.int64),
                       classes=wl.classes, append=int(wl.steps[0].ctx[0] - wl.ctx0[0]),
                       group=group)
    wl2 = hs_gen.build_dynamic(spec, d, wl.n_blocks, dec.p.cfg.num_host_blocks)
    assert mp == wl2.max_pages
    _same_edits(wl, wl2)
