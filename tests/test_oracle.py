"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these expectations comes from the oracle itself or from the GPU
library: they are hand-derived worked examples, a textbook LRU, an exhaustive
enumeration of the declarative conditions, closed forms, a library routine
(torch.index_select) and the synthetic content every row must hold.
"""

from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import hs_gen
import oracle
from hs_gen import rng
from harness import OracleRun, expected_content, run_tiny, tiny_instance
from models import TextbookLRU, declarative_solutions, sequential_resolve

ROW = hs_gen.ROW_BYTES


# --------------------------------------------------------------------------
# input generator sanity (shared by both sides, so it is pinned first)

def test_splitmix64_published_vector():
    # splitmix64 seeded with 0: first outputs as published with the algorithm
    assert rng.splitmix64(0) == 0xE220A8397B1DCDAF
    assert rng.splitmix64(rng.GAMMA) == 0x6E789E6AA1B965F4
    assert rng.splitmix64(2 * rng.GAMMA & rng.MASK64) == 0x06C45D188009454F


def test_rng_implementations_agree():
    xs = [0, 1, 2, 12345, (1 << 63) + 17, rng.MASK64, 0x0123456789ABCDEF]
    ref = [rng.splitmix64(x) for x in xs]
    assert rng.splitmix64_np(np.array(xs, dtype=np.uint64)).tolist() == ref
    t = torch.tensor([x - (1 << 64) if x >= (1 << 63) else x for x in xs], dtype=torch.int64)
    got = [(v + (1 << 64)) % (1 << 64) for v in rng.splitmix64_torch(t).tolist()]
    assert got == ref


def test_content_numpy_torch_agree():
    lay = np.array([0, 3, 15, 1])
    src = np.array([0, 5, 1, 64])
    tok = np.array([0, 74159, 999_999, 12])
    a = hs_gen.content_np(lay, src, tok)
    b = hs_gen.content_torch(torch.from_numpy(lay), torch.from_numpy(src),
                             torch.from_numpy(tok)).numpy()
    assert a.shape == (4, ROW) and np.array_equal(a, b)
    assert len({bytes(r) for r in a}) == 4


# --------------------------------------------------------------------------
# hand-worked example (derived by hand from the resolve steps; every number
# below can be rechecked with pencil and paper)
#
# page 4, ctx 24 (pages 0..5), one request, one layer, 8 hot slots.
# hot_blocks [9, 6]: slots 0..3 -> rows 36..39, slots 4..7 -> rows 24..27.
# block table [-1,-1,-1,-1,7,2]: page 4 -> rows 28..31, page 5 -> rows 8..11.
# host block table [3,0,5,1,4,2]: page p's token o is host row hbt[p]*4 + o.

def _ids(pool_rows_bytes):
    return [int(np.frombuffer(r[:4].tobytes(), np.int32)[0]) for r in pool_rows_bytes]


def test_worked_example_steps():
    inst = tiny_instance()
    pool0 = inst["pool"].copy()

    # step 1 (stamp 1): 21 and 17 are resident (rows 9, 29); misses 2,5,9,13
    # fill the empty slots 0..3 in ascending order.
    rows, stats, out = run_tiny(inst, [21, 5, 13, 2, 17, 9], 1)
    assert rows.ravel().tolist() == [9, 37, 39, 36, 29, 38]
    assert inst["tok"].ravel().tolist() == [2, 5, 9, 13, -1, -1, -1, -1]
    assert inst["stp"].ravel().tolist() == [1, 1, 1, 1, 0, 0, 0, 0]
    assert stats.ravel()[:3].tolist() == [2, 0, 4]
    # copies host row -> pool row: 14->36, 1->37, 21->38, 5->39 (host rows
    # carry their own index, tagged 0x40)
    for host_row, pool_row in [(14, 36), (1, 37), (21, 38), (5, 39)]:
        assert np.array_equal(inst["pool"][0, pool_row], inst["host"][0, host_row])
    # the gathered rows are the pool rows after the copies
    assert _ids(out.reshape(-1, ROW)) == [9, 1, 5, 14, 29, 21]

    # step 2 (stamp 2): 9 and 13 hit (slots 2, 3); misses 1, 6, 14 take the
    # never-used slots 4, 5, 6 (stamp 0 sorts before stamp 1).
    rows, stats, _ = run_tiny(inst, [9, 1, 22, 13, 6, 14], 2)
    assert rows.ravel().tolist() == [38, 24, 10, 39, 25, 26]
    assert inst["tok"].ravel().tolist() == [2, 5, 9, 13, 1, 6, 14, -1]
    assert inst["stp"].ravel().tolist() == [1, 1, 2, 2, 2, 2, 2, 0]
    assert stats.ravel()[:3].tolist() == [1, 2, 3]
    for host_row, pool_row in [(13, 24), (2, 25), (6, 26)]:
        assert np.array_equal(inst["pool"][0, pool_row], inst["host"][0, host_row])

    # step 3 (stamp 3): page 4 becomes a null placeholder first (its host copy
    # is host block 4).  2 and 6 hit; misses 3, 10, 17 take slot 7 (stamp 0),
    # slot 1 (stamp 1, evicting 5) and slot 2 (stamp 2, lowest slot, evicting 9).
    inst["bt"][0, 4] = -1
    rows, stats, _ = run_tiny(inst, [17, 2, 10, 6, 20, 3], 3)
    assert rows.ravel().tolist() == [38, 36, 37, 25, 8, 27]
    assert inst["tok"].ravel().tolist() == [2, 10, 17, 13, 1, 6, 14, 3]
    assert inst["stp"].ravel().tolist() == [3, 3, 3, 2, 2, 3, 2, 3]
    assert stats.ravel()[:3].tolist() == [1, 2, 3]
    for host_row, pool_row in [(15, 27), (22, 37), (17, 38)]:
        assert np.array_equal(inst["pool"][0, pool_row], inst["host"][0, host_row])

    # step 4 (stamp 4): replay of step 3's list -- every non-resident token
    # hits, nothing is copied, the touched slots take stamp 4.
    before = inst["pool"].copy()
    rows, stats, _ = run_tiny(inst, [17, 2, 10, 6, 20, 3], 4)
    assert rows.ravel().tolist() == [38, 36, 37, 25, 8, 27]
    assert inst["tok"].ravel().tolist() == [2, 10, 17, 13, 1, 6, 14, 3]
    assert inst["stp"].ravel().tolist() == [4, 4, 4, 2, 2, 4, 2, 4]
    assert stats.ravel()[:3].tolist() == [1, 5, 0]
    assert np.array_equal(before, inst["pool"])
    # rows outside the hot blocks (9, 6) were never written
    hot_rows = set(range(36, 40)) | set(range(24, 28))
    for r in range(pool0.shape[1]):
        if r not in hot_rows:
            assert np.array_equal(pool0[0, r], inst["pool"][0, r])


def test_worked_example_plan_overflow_invalid():
    # plan over 2 positions x 3 tokens from the state after step 1
    inst = tiny_instance()
    run_tiny(inst, [21, 5, 13, 2, 17, 9], 1)
    rows, stats, _ = run_tiny(inst, np.array([[9, 1, 22], [13, 1, 6]]), 2)
    assert rows.tolist() == [[[[38, 24, 10], [39, 24, 25]]]]
    assert inst["tok"].ravel().tolist() == [2, 5, 9, 13, 1, 6, -1, -1]
    assert inst["stp"].ravel().tolist() == [1, 1, 2, 2, 2, 2, 0, 0]
    assert stats.ravel().tolist() == [1, 2, 2, 0, 0, 0, 1, 0]

    # overflow: 4 slots (hot block 9 only), 3 misses but only 2 non-hit slots
    inst = tiny_instance(C=4, hot_blocks=(9,))
    run_tiny(inst, [21, 5, 13, 2, 17, 9], 1)
    rows, stats, _ = run_tiny(inst, np.array([[9, 1, 22], [13, 6, 14]]), 2)
    assert rows.tolist() == [[[[38, 36, 10], [39, 37, -2]]]]
    assert inst["tok"].ravel().tolist() == [1, 6, 9, 13]
    assert inst["stp"].ravel().tolist() == [2, 2, 2, 2]
    assert stats.ravel().tolist() == [1, 2, 2, 1, 0, 0, 0, 0]

    # padding, out-of-range, and a hit that wins over a missing host copy
    inst = tiny_instance(hbt=(3, 0, -1, 1, 4, 2))
    run_tiny(inst, [21, 5, 13, 2, 17], 1)
    inst["tok"][0, 0, 2] = 9  # 9 sits in slot 2 although page 2 has no host copy
    inst["stp"][0, 0, 2] = 1
    rows, stats, out = run_tiny(inst, [-1, 30, 9, 10, -5, 21], 2)
    assert rows.ravel().tolist() == [-1, -3, 38, -3, -3, 9]
    assert stats.ravel().tolist() == [1, 1, 0, 0, 3, 1, 0, 0]
    o = out.reshape(-1, ROW)
    assert not o[[0, 1, 3, 4]].any()


# --------------------------------------------------------------------------
# K = 1 reduces to a textbook LRU cache

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_single_token_lists_are_textbook_lru(seed):
    page, C = 4, 8
    universe = 40                       # tokens 0..39, pages 0..9, none resident
    inst = tiny_instance(page=page, ctx=universe, C=C, hot_blocks=(11, 3),
                         bt=(-1,) * 10, hbt=tuple(range(10)), n_blocks=12, n_host=10)
    lru = TextbookLRU(C)
    r = random.Random(seed)
    hot_row = lambda q: (11, 3)[q // page] * page + q % page
    for step in range(1, 400):
        t = r.randrange(universe) if r.random() < 0.6 else r.randrange(12)
        kind, slot, _ = lru.access(t)
        rows, stats, _ = run_tiny(inst, [t], step)
        assert rows.ravel().tolist() == [hot_row(slot)]
        assert stats.ravel()[1:3].tolist() == ([1, 0] if kind == "hit" else [0, 1])
        held = {tk: q for tk, q in lru.order.items()}
        for q in range(C):
            tk = int(inst["tok"][0, 0, q])
            if tk >= 0:
                assert held[tk] == q


# --------------------------------------------------------------------------
# exhaustive enumeration of the declarative conditions on tiny inputs

@pytest.mark.parametrize("seed", range(40))
def test_victims_are_the_unique_declarative_solution(seed):
    r = random.Random(1000 + seed)
    page = 2
    C = r.choice([2, 4, 6])
    n_pages = 8
    ctx = page * n_pages
    inst = tiny_instance(page=page, ctx=ctx, C=C,
                         hot_blocks=tuple(20 + i for i in range(C // page)),
                         bt=tuple(-1 if r.random() < 0.7 else 10 + p for p in range(n_pages)),
                         hbt=tuple(p if r.random() < 0.9 else -1 for p in range(n_pages)),
                         n_blocks=20 + C // page, n_host=n_pages)
    # a random pre-state: distinct tokens in some slots, stamps in {0,1,2}
    toks = r.sample(range(ctx), C)
    for q in range(C):
        if r.random() < 0.6:
            inst["tok"][0, 0, q] = toks[q]
            inst["stp"][0, 0, q] = r.choice([1, 2])
        else:
            inst["stp"][0, 0, q] = r.choice([0, 0, 1])
    tok0 = inst["tok"].ravel().tolist()
    stp0 = inst["stp"].ravel().tolist()
    lst = [r.randrange(-1, ctx) for _ in range(r.choice([1, 2, 3, 4]))]
    rows, stats, _ = run_tiny(inst, lst, 3)

    bt = inst["bt"][0].tolist()
    hbt = inst["hbt"][0].tolist()
    nonres = sorted({t for t in lst if 0 <= t < ctx and bt[t // page] < 0})
    where = {tok0[q]: q for q in range(C) if tok0[q] >= 0}
    hit_slots = {where[t] for t in nonres if t in where}
    misses = [t for t in nonres if t not in where and hbt[t // page] >= 0]
    sols = declarative_solutions(hit_slots, misses, list(range(C)),
                                 {q: stp0[q] for q in range(C)})
    assert len(sols) == 1, sols
    assign = sols[0]
    hot_row = lambda q: (20 + q // page) * page + q % page
    for t, row in zip(lst, rows.ravel().tolist()):
        if t in assign:
            assert row == hot_row(assign[t])
        elif t in misses:
            assert row == -2
    for t, q in assign.items():
        assert inst["tok"][0, 0, q] == t and inst["stp"][0, 0, q] == 3


@pytest.mark.parametrize("seed", range(60))
def test_matches_sequential_restatement(seed):
    r = random.Random(seed)
    page = r.choice([2, 4])
    n_pages = r.choice([4, 6, 8])
    ctx = page * n_pages - r.randrange(page)
    C = page * r.choice([1, 2, 3])
    inst = tiny_instance(page=page, ctx=ctx, C=C,
                         hot_blocks=tuple(r.sample(range(30, 40), C // page)),
                         bt=tuple(-1 if r.random() < 0.6 else r.randrange(10, 30)
                                  for _ in range(n_pages)),
                         hbt=tuple(-1 if r.random() < 0.15 else p for p in range(n_pages)),
                         n_blocks=40, n_host=n_pages)
    stamp = 0
    for _ in range(6):
        stamp += r.choice([1, 1, 2])
        lst = [r.randrange(-2, ctx + 2) for _ in range(r.randrange(1, 2 * C + 2))]
        tok0 = inst["tok"].ravel().tolist()
        stp0 = inst["stp"].ravel().tolist()
        pool0 = inst["pool"].copy()
        exp_rows, exp_tok, exp_stp, copies = sequential_resolve(
            lst, ctx, page, inst["bt"][0].tolist(), inst["hbt"][0].tolist(),
            inst["hot"][0].tolist(), tok0, stp0, stamp, pool_blocks=40, host_blocks=n_pages)
        rows, stats, out = run_tiny(inst, lst, stamp)
        assert rows.ravel().tolist() == exp_rows
        assert inst["tok"].ravel().tolist() == exp_tok
        assert inst["stp"].ravel().tolist() == exp_stp
        exp_pool = pool0.copy()
        for host_row, pool_row in copies:
            exp_pool[0, pool_row] = inst["host"][0, host_row]
        assert np.array_equal(exp_pool, inst["pool"])
        assert int(stats.sum()) == len(lst)


# --------------------------------------------------------------------------
# closed forms

def test_empty_buffer_fills_slots_in_token_order():
    # no resident page, empty hot buffer, distinct misses <= C: the j-th
    # smallest token lands in slot j
    page, C = 64, 512
    r = np.random.default_rng(5)
    hot = r.permutation(100)[:C // page] + 200
    ctx = 64 * 40
    inst = tiny_instance(page=page, ctx=ctx, C=C, hot_blocks=tuple(hot.tolist()),
                         bt=(-1,) * 40, hbt=tuple(range(40)), n_blocks=300, n_host=40)
    lst = r.choice(ctx, size=300, replace=False)
    rows, stats, _ = run_tiny(inst, lst, 1)
    rank = np.argsort(np.argsort(lst))
    exp = hot[rank // page] * page + rank % page
    assert rows.ravel().tolist() == exp.tolist()
    assert stats.ravel().tolist() == [0, 0, 300, 0, 0, 0, 0, 0]


def test_gather_is_index_select():
    r = np.random.default_rng(3)
    pool = r.integers(0, 256, size=(3, 640, ROW), dtype=np.uint8)
    rows = r.integers(-5, 700, size=(2, 3, 100)).astype(np.int32)
    out = oracle.gather(pool, rows)
    tp = torch.from_numpy(pool)
    for layer in range(3):
        idx = torch.from_numpy(rows[:, layer].ravel().astype(np.int64))
        ok = (idx >= 0) & (idx < 640)
        exp = torch.index_select(tp[layer], 0, torch.where(ok, idx, 0))
        exp[~ok] = 0
        assert np.array_equal(out[:, layer].reshape(-1, ROW), exp.numpy())


def test_offload_copies_every_layer_and_leaves_pool():
    r = np.random.default_rng(4)
    L = 3
    pool = r.integers(0, 256, size=(L, 64 * 10, ROW), dtype=np.uint8)
    host = r.integers(0, 256, size=(L, 64 * 6, ROW), dtype=np.uint8)
    pool0, host0 = pool.copy(), host.copy()
    pairs = np.array([[7, 2], [1, 5], [9, 0], [12, 1], [3, 9]], dtype=np.int32)  # last two out of range
    oracle.offload(pool, host, pairs)
    assert np.array_equal(pool, pool0)
    exp = host0.copy()
    for db, hb in [(7, 2), (1, 5), (9, 0)]:
        exp[:, hb * 64:(hb + 1) * 64] = pool0[:, db * 64:(db + 1) * 64]
    assert np.array_equal(host, exp)


# --------------------------------------------------------------------------
# whole synthetic workloads: content and invariants

def _check_invariants(run: OracleRun, step, rows, stats, out, pool_before, tok_before,
                      stp_before):
    wl = run.wl
    N = wl.P * wl.K
    assert np.array_equal(stats.sum(axis=2), np.full((wl.R, wl.L), N))
    # every gathered row is the content of its token (or zeros)
    assert np.array_equal(out, expected_content(wl, step.topk, rows))
    page = hs_gen.PAGE
    for r in range(wl.R):
        hot_rows = (run.hot[r][:, None] * page + np.arange(page)[None, :]).ravel()
        for layer in range(wl.L):
            tok, stp = run.tok[r, layer], run.stp[r, layer]
            live = tok[tok >= 0]
            assert live.size == np.unique(live).size          # no token in two slots
            assert np.all((stp == 0) == (tok < 0))             # stamp 0 <=> empty
            changed = (tok != tok_before[r, layer])
            touched = stp == step.stamp
            assert np.all(touched[changed])                    # every fill is stamped
            # rows of slots that did not change hands were not rewritten
            same = hot_rows[~changed]
            assert np.array_equal(run.pool[layer, same], pool_before[layer, same])
    # nothing outside the hot blocks was written (the resident tail included)
    all_hot = (run.hot.reshape(-1)[:, None] * page + np.arange(page)[None, :]).ravel()
    mask = np.ones(wl.pool_rows, dtype=bool)
    mask[all_hot] = False
    assert np.array_equal(run.pool[:, mask], pool_before[:, mask])


def test_tiny_workload_invariants():
    wl = hs_gen.tiny()
    run = OracleRun(wl)
    for step in wl.steps:
        run.pre(step)
        pb, tb, sb = run.pool.copy(), run.tok.copy(), run.stp.copy()
        rows, stats, out = run.resolve(step)
        _check_invariants(run, step, rows, stats, out, pb, tb, sb)
        run.post(step)
    # replaying the last list with the same stamp changes no state
    tb, sb, pb = run.tok.copy(), run.stp.copy(), run.pool.copy()
    rows2, stats2, _ = run.resolve(wl.steps[-1])
    assert np.array_equal(tb, run.tok) and np.array_equal(sb, run.stp)
    assert np.array_equal(pb, run.pool)
    assert stats2[..., 2].sum() == 0


def test_mixed_decode_reduced_invariants_and_offload():
    wl = hs_gen.mixed_decode(R=3)
    run = OracleRun(wl)
    seen_hits = 0
    for step in wl.steps:
        run.pre(step)
        pb, tb, sb = run.pool.copy(), run.tok.copy(), run.stp.copy()
        rows, stats, out = run.resolve(step)
        _check_invariants(run, step, rows, stats, out, pb, tb, sb)
        seen_hits += int(stats[..., 1].sum())
        host_before = run.host.copy()
        run.post(step)
        for db, hb in step.offload:
            # the proactive copy holds the page's content; the device pool is unchanged
            assert np.array_equal(run.host[:, hb * 64:(hb + 1) * 64], run.pool[:, db * 64:(db + 1) * 64])
        untouched = np.ones(wl.host_rows, dtype=bool)
        for _, hb in step.offload:
            untouched[hb * 64:(hb + 1) * 64] = False
        assert np.array_equal(run.host[:, untouched], host_before[:, untouched])
    assert seen_hits > 0
    assert sum(s.offload.shape[0] for s in wl.steps) == 3


@pytest.mark.parametrize("G", [1, 2])
def test_blocked_oracle_run_equals_whole_batch(G):
    """The tests' threaded driver of the oracle (blocks of requests on threads
    of their own, for the full-size batches) gives the whole batch's result:
    request-layers are independent and their hot blocks disjoint."""
    spec = hs_gen.Spec(name="blocked", seed=21, R=7, L=2, K=256, C=512, steps=3,
                       ctx0=np.array([9000, 20000, 5000, 7000, 12000, 3000, 16000]),
                       classes=np.array([1, 2, 0, 1, 1, 2, 1], np.int8), append=70, P=2, pos_keep=160,
                       group=G)
    wl = hs_gen.build(spec)
    whole, blocked = OracleRun(wl), OracleRun(wl, threads=3)
    for step in wl.steps:
        for run in (whole, blocked):
            run.pre(step)
        a, b = whole.resolve(step), blocked.resolve(step)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        for run in (whole, blocked):
            run.post(step)
        assert np.array_equal(whole.tok, blocked.tok) and np.array_equal(whole.stp, blocked.stp)
        assert np.array_equal(whole.pool, blocked.pool)
        assert np.array_equal(whole.host, blocked.host)


def test_plan_equals_resolve_of_concatenation():
    wl = hs_gen.build(hs_gen.Spec(name="plan", seed=11, R=3, L=2, K=128, C=512, steps=3,
                                  ctx0=np.array([9000, 20000, 5000]),
                                  classes=np.array([0, 1, 2], np.int8), P=3, pos_keep=96,
                                  shared_src=True))
    a, b = OracleRun(wl), OracleRun(wl)
    for step in wl.steps:
        a.pre(step)
        b.pre(step)
        ra, sa, oa = a.resolve(step)
        flat = step.topk.reshape(wl.R, wl.L, -1)
        rb, sb, ob = b.resolve(step, topk=flat)
        assert np.array_equal(ra.reshape(rb.shape), rb)
        assert np.array_equal(sa, sb)
        assert np.array_equal(a.tok, b.tok) and np.array_equal(a.stp, b.stp)
        assert np.array_equal(oa, expected_content(wl, step.topk, ra))


# --------------------------------------------------------------------------
# grouped resolve (IndexShare: layers of a group share one top-K list)

def _grouped_spec(G, seed=77, L=4):
    return hs_gen.Spec(name="grouped_small", seed=seed, R=3, L=L, K=256, C=512, steps=4,
                       ctx0=np.array([4096, 3000, 5000]), classes=np.array([1, 1, 2], np.int8),
                       tail_frac=0.25, mix=(0.5, 0.2, 0.3), group=G)


@pytest.mark.parametrize("G", [2, 4])
def test_grouped_equals_per_layer_resolve(G):
    """A grouped resolve is the per-layer resolve of every layer of the group on
    the group's list, from the group's state: same rows, stats, final states
    (every layer ends with the group's state), pools and gathered rows."""
    wl = hs_gen.build(_grouped_spec(G))
    grp = OracleRun(wl)
    flat = OracleRun(wl)
    flat.tok = np.repeat(grp.tok, G, axis=1)
    flat.stp = np.repeat(grp.stp, G, axis=1)
    moved = 0
    for step in wl.steps:
        grp.pre(step)
        flat.pre(step)
        g_rows, g_stats, g_out = grp.resolve(step)
        rep = np.ascontiguousarray(np.repeat(step.topk, G, axis=1))
        f_rows, f_stats, f_out = oracle.resolve(flat.pool, flat.host, flat.bt, flat.hbt,
                                                flat.ctx, flat.hot, flat.tok, flat.stp, rep,
                                                step.stamp, True)
        assert np.array_equal(f_rows, np.repeat(g_rows, G, axis=1))
        assert np.array_equal(f_stats, np.repeat(g_stats, G, axis=1))
        assert np.array_equal(flat.tok, np.repeat(grp.tok, G, axis=1))
        assert np.array_equal(flat.stp, np.repeat(grp.stp, G, axis=1))
        assert np.array_equal(flat.pool, grp.pool)
        assert np.array_equal(f_out, g_out)
        moved += int(g_stats[..., 2].sum())
        grp.post(step)
        flat.post(step)
        assert np.array_equal(flat.host, grp.host)
    assert moved > 0


def test_grouped_rows_hold_each_layers_content():
    """Every gathered row of every layer holds that layer's content of the token."""
    wl = hs_gen.build(_grouped_spec(4))
    run = OracleRun(wl)
    for step in wl.steps:
        run.pre(step)
        rows, stats, out = run.resolve(step)
        assert out.shape[1] == wl.L
        assert np.array_equal(out, expected_content(wl, step.topk, rows))
        run.post(step)


def test_grouped_with_one_layer_per_group_is_resolve():
    wl = hs_gen.build(_grouped_spec(1))
    a, b = OracleRun(wl), OracleRun(wl)
    for step in wl.steps[:2]:
        a.pre(step)
        b.pre(step)
        ra = a.resolve(step)
        rb = oracle.resolve_grouped(b.pool, b.host, b.bt, b.hbt, b.ctx, b.hot, b.tok, b.stp,
                                    np.ascontiguousarray(step.topk), step.stamp, 1, True)
        for x, y in zip(ra, rb):
            assert np.array_equal(x, y)
        assert np.array_equal(a.pool, b.pool) and np.array_equal(a.tok, b.tok)


def test_page_touch_worked_example():
    """Page coldness by hand (page 4): request 0 (context 12) selects tokens
    3 (page 0), 6 (page 1) and 9 (page 2); 12 lies past the context and -1
    is padding, so page 3 keeps its old stamp.  Request 1 (context 16)
    selects 12 and 15 (page 3); 16 is past the context, -5 invalid."""
    use = np.array([[7, 7, 7, 7], [1, 2, 3, 4]], np.uint32)
    topk = np.array([[3, 9, 12, -1, 6, -1], [15, 16, -5, 12, -1, -1]], np.int32)
    oracle.page_touch(np.array([12, 16], np.int32), topk, 9, use, page=4)
    assert use.tolist() == [[9, 9, 9, 7], [1, 2, 3, 9]]


def test_page_touch_is_the_set_of_selected_pages():
    """On random lists (padding, out-of-range and past-the-table tokens
    included), exactly the pages holding a selected context token carry the
    new stamp, and every other word is unchanged."""
    rs = np.random.default_rng(5)
    R, max_pages, E = 12, 40, 24
    PAGE = hs_gen.PAGE
    ctx = rs.integers(1, 45 * PAGE, size=R).astype(np.int32)   # some contexts exceed the table
    topk = rs.integers(-3, 46 * PAGE, size=(R, 2, E // 2)).astype(np.int32)
    # the context's last token and the first one past it, on every request
    topk[:, 0, 0] = ctx - 1
    topk[:, 1, 0] = ctx
    old = rs.integers(1, 1000, size=(R, max_pages)).astype(np.uint32)
    use = old.copy()
    oracle.page_touch(ctx, topk, 4242, use)
    for r in range(R):
        t = topk[r].ravel()
        t = t[(t >= 0) & (t < ctx[r])]
        pages = set((t // PAGE).tolist()) & set(range(max_pages))
        touched = set(np.nonzero(use[r] == 4242)[0].tolist())
        assert touched == pages
        keep = np.ones(max_pages, bool)
        keep[list(pages)] = False
        assert np.array_equal(use[r][keep], old[r][keep])
