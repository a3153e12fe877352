"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit-exact.

Every comparison is element by element on the same seeded inputs: row ids,
stats, hot-buffer tokens and stamps, every byte of the hot-slot rows, every
gathered byte, and the host pool after each prefix offload.  The five
workloads run at their full sizes with every request compared; quicker
sampled forms of the two largest (64 x 16 request-layers, 128 requests x 4
positions) add content checks and the staged paths (request-layers are
independent, so a subset of requests resolves exactly as inside the batch).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import hs_gen
import stages
from harness import OracleRun, expected_content, policy_workload

pytestmark = pytest.mark.gpu

ROW = hs_gen.ROW_BYTES
PAGE = hs_gen.PAGE


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import serving_memory_tier_amd as hs
    import os
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hs.lib()


def _hot_rows(hot_blocks: np.ndarray) -> np.ndarray:
    return (hot_blocks.reshape(-1)[:, None] * PAGE + np.arange(PAGE)[None, :]).ravel()


def _say(msg: str) -> None:
    print(msg, flush=True)


def _equal_by_layer(dev_pool, ora_pool, rows=None) -> bool:
    """Pool planes compared one layer at a time (the largest batches hold
    tens of GB), optionally only the given rows."""
    idx = None if rows is None else torch.from_numpy(rows).cuda()
    for layer in range(ora_pool.shape[0]):
        d = dev_pool[layer] if idx is None else dev_pool[layer, idx]
        o = ora_pool[layer] if rows is None else ora_pool[layer, rows]
        if not np.array_equal(d.cpu().numpy(), o):
            return False
    return True


def run_parity(wl, requests=None, n_steps=None, hit_replay=False, fused_plan=False,
               check_content=True, mode="call", gather=True, threads=8):
    from serving_memory_tier_amd.runner import DeviceRun

    dev = DeviceRun(wl)
    dev.upload_steps()
    ora = OracleRun(wl, requests, content_device="cuda", threads=threads)
    req = torch.from_numpy(ora.req).cuda()
    steps = wl.steps if n_steps is None else wl.steps[:n_steps]
    totals = np.zeros(8, dtype=np.int64)
    try:
        for i, step in enumerate(steps):
            _say(f"[parity] {wl.name} step {i} stamp {step.stamp}")
            dev.pre(i)
            ora.pre(step)
            if fused_plan:
                dev.plan_step(i)
            elif mode == "call":
                dev.resolve(i, gather=gather)
            else:
                stages.run(mode, dev.layout, dev.batch, dev.topk[i], wl.P, wl.K, step.stamp,
                           dev.rows, dev.out, dev.stats)
            torch.cuda.synchronize()
            rows, stats, out = ora.resolve(step, gather=gather)
            totals += stats.sum(axis=(0, 1))
            assert np.array_equal(dev.rows[req].cpu().numpy(), rows), f"row ids, step {i}"
            assert np.array_equal(dev.stats[req].cpu().numpy(), stats), f"stats, step {i}"
            assert np.array_equal(dev.tok[req].cpu().numpy(), ora.tok), f"slot tokens, step {i}"
            assert np.array_equal(dev.stp[req].cpu().numpy().view(np.uint32), ora.stp), \
                f"slot stamps, step {i}"
            if gather:
                g_out = dev.out[req].cpu().numpy()
                assert np.array_equal(g_out, out), f"gathered rows, step {i}"
            if gather and check_content:
                assert np.array_equal(g_out, expected_content(wl, step.topk[ora.req], rows,
                                                              ora.req)), f"content, step {i}"
            # the hot slots' rows (leases can move between steps)
            hot_rows = _hot_rows(ora.hot[ora.hot >= 0])
            assert _equal_by_layer(dev.pool, ora.pool, hot_rows), f"hot rows, step {i}"
            if hit_replay:
                # the same lists with the same stamp: every non-resident token
                # is now a hit, nothing is copied, the state does not move
                tok0, stp0 = dev.tok.clone(), dev.stp.clone()
                dev.resolve(i)
                torch.cuda.synchronize()
                rows2, stats2, out2 = ora.resolve(step)
                assert np.array_equal(dev.rows[req].cpu().numpy(), rows2)
                assert np.array_equal(dev.stats[req].cpu().numpy(), stats2)
                assert np.array_equal(dev.out[req].cpu().numpy(), out2)
                assert int(stats2[..., 2].sum()) == 0
                assert torch.equal(tok0, dev.tok) and torch.equal(stp0, dev.stp)
            if not fused_plan:
                dev.post(i)
            ora.post(step)
            pr = ora.pairs(step)
            if pr.shape[0]:
                torch.cuda.synchronize()
                hb = torch.from_numpy((pr[:, 1].astype(np.int64)[:, None] * PAGE +
                                       np.arange(PAGE)[None, :]).ravel())
                assert np.array_equal(dev.host[:, hb].numpy(), ora.host[:, hb.numpy()]), \
                    f"host pool after offload, step {i}"
        torch.cuda.synchronize()
        if requests is None:
            assert _equal_by_layer(dev.pool, ora.pool), "final pool"
            assert np.array_equal(dev.host.numpy(), ora.host), "final host pool"
    finally:
        dev.close()
    return totals


def test_tiny():
    totals = run_parity(hs_gen.tiny(), hit_replay=True)
    assert totals[2] > 0 and totals[1] > 0


def test_mixed_decode_full():
    totals = run_parity(hs_gen.mixed_decode(), hit_replay=True)
    _say(f"[parity] mixed_decode totals {totals.tolist()}")
    assert totals[1] > 0 and totals[2] > 0 and totals[0] > 0


@pytest.mark.parametrize("mode", ["serial", "staged", "in_place"])
def test_mixed_decode_stages(mode):
    totals = run_parity(hs_gen.mixed_decode(steps=6), mode=mode, gather=mode != "in_place")
    assert totals[2] > 0


def test_no_residency_full():
    totals = run_parity(hs_gen.no_residency())
    _say(f"[parity] no_residency totals {totals.tolist()}")
    assert totals[2] >= 8 * 2048 * 0.99


@pytest.mark.timeout(900)
def test_mixed_state_full():
    """The mixed-state batch in full: all 128 requests (full, mixed and
    no residency), 4 positions x 2048 per step resolved as one plan with its
    gather and the offload of the pages each step completes, 16 steps; the
    final pool and host pool compared whole."""
    totals = run_parity(hs_gen.mixed_state(), fused_plan=True, check_content=False, threads=16)
    _say(f"[parity] mixed_state totals {totals.tolist()}")
    assert totals[0] > 0 and totals[1] > 0 and totals[2] > 0


@pytest.mark.timeout(900)
def test_multi_layer_full():
    """The multi-layer batch in full: 64 requests x 16 layers in one launch,
    13 turns of +753 tokens with the tail moving, and after every turn the
    offload of the completed pages of all 16 layers in one launch; every
    request's rows, state and gathered bytes per turn, the host pool after
    each offload, and the final pool and host pool whole."""
    totals = run_parity(hs_gen.multi_layer(), check_content=False, threads=16)
    _say(f"[parity] multi_layer totals {totals.tolist()}")
    assert totals[0] > 0 and totals[1] > 0 and totals[2] > 0


def test_mixed_state_full_sampled():
    wl = hs_gen.mixed_state()
    # two requests of each residency class plus the largest and smallest context
    sample = []
    for c in (0, 1, 2):
        sample += list(np.nonzero(wl.classes == c)[0][:3])
    sample += [int(np.argmax(wl.ctx0)), int(np.argmin(wl.ctx0))]
    sample = sorted(set(int(s) for s in sample))
    run_parity(wl, requests=sample, fused_plan=True)


def test_mtp_state_full_sampled():
    """The speculative-decoding sizing at full size: 128 requests, a
    4-position plan of 2048 each, 10,240 hot slots per request."""
    wl = hs_gen.mtp_state(steps=8)
    assert wl.C == 10240 and wl.P * wl.K == 8192
    sample = []
    for c in (0, 1, 2):
        sample += list(np.nonzero(wl.classes == c)[0][:2])
    sample += [int(np.argmax(wl.ctx0))]
    sample = sorted(set(int(s) for s in sample))
    totals = run_parity(wl, requests=sample, fused_plan=True)
    assert totals[3] == 0          # the plan's union always fits: no overflow
    assert totals[1] > 0 and totals[2] > 0


def test_multi_layer_full_sampled():
    wl = hs_gen.multi_layer(turns=4)
    run_parity(wl, requests=[0, 17, 63], fused_plan=False)


@pytest.mark.parametrize("mode", ["serial", "staged", "in_place"])
def test_mixed_state_stages_sampled(mode):
    wl = hs_gen.mixed_state(steps=4)
    run_parity(wl, requests=[0, 1, 64, 127], mode=mode, gather=mode != "in_place")


@pytest.mark.parametrize("gather", [True, False])
def test_grouped_decode(gather):
    """Layers sharing a top-K list (IndexShare): 32 requests x 4 layers in one
    group, resolved once per group, every layer's rows moved."""
    wl = hs_gen.grouped_decode(steps=6)
    if gather:
        totals = run_parity(wl)
    else:
        totals = run_parity(wl, gather=False)
    assert totals[1] > 0 and totals[2] > 0


def test_determinism_repeat():
    """Two runs of the same steps give bitwise identical results."""
    from serving_memory_tier_amd.runner import DeviceRun

    wl = hs_gen.mixed_decode(R=8, steps=4)
    res = []
    for _ in range(2):
        dev = DeviceRun(wl)
        outs = []
        for i in range(len(wl.steps)):
            dev.pre(i)
            dev.resolve(i)
            outs.append((dev.rows.clone(), dev.stats.clone(), dev.out.clone()))
        torch.cuda.synchronize()
        res.append((outs, dev.tok.clone(), dev.stp.clone(), dev.pool.clone()))
        dev.close()
    for (a, b) in zip(res[0][0], res[1][0]):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    for x, y in zip(res[0][1:], res[1][1:]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("block", [1, 5, 8])
def test_launch_shape_independence(block):
    """No byte depends on the launch shape: the fused launch sizes its gather
    workgroups (and so every gather range) from the request-layers it holds
    and the chip's occupancy.  The same mixed-decode steps resolved as one
    batch of 32 requests and as consecutive sub-batches of ``block``
    requests (leading slices of the same tables, state and outputs, so every
    launch has another shape) give identical rows, stats, gathered bytes,
    state and pool, step after step, hit replays included."""
    import serving_memory_tier_amd as hs
    from serving_memory_tier_amd.runner import DeviceRun

    wl = hs_gen.mixed_decode(steps=5)
    a, b = DeviceRun(wl), DeviceRun(wl)
    try:
        for d in (a, b):
            d.upload_steps()
        for i, step in enumerate(wl.steps):
            _say(f"[parity] launch shapes, block {block}, step {i}")
            for stamp in (step.stamp, step.stamp):         # the step, then its hit replay
                a.pre(i)
                a.resolve(i, stamp=stamp)
                b.pre(i)
                for r0 in range(0, wl.R, block):
                    r1 = min(wl.R, r0 + block)
                    sub = hs.batch_of(r1 - r0, wl.max_pages, b.pool, b.host_pool, b.bt[r0:r1],
                                      b.hbt[r0:r1], b.ctx[r0:r1], b.hot[r0:r1], b.tok[r0:r1],
                                      b.stp[r0:r1])
                    hs.hs_resolve(b.layout, sub, b.topk[i][r0:r1], wl.K, stamp, b.rows[r0:r1],
                                  b.out[r0:r1], b.stats[r0:r1])
                torch.cuda.synchronize()
                for x, y in ((a.rows, b.rows), (a.stats, b.stats), (a.tok, b.tok),
                             (a.stp, b.stp), (a.out, b.out), (a.pool, b.pool)):
                    assert torch.equal(x, y), f"step {i}"
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("group", [1, 2])
def test_policy_driven_small(group):
    """Residency decided step by step by the host policy: blocks freed by
    evictions are reused for new pages and hot leases, leases are granted
    mid-run (the request's hot buffer starts empty), and host copies the
    previous step queued back the pages nulled now."""
    wl, dec = policy_workload(group=group, L=2 * group)
    assert dec.evicted > 0 and dec.leased > len(wl.steps[0].ctx) // 2
    totals = run_parity(wl)
    assert totals[2] > 0 and totals[1] > 0


def _policy_sweep_params(seed):
    """Random policy-driven workloads: batch, layers (in groups of 1 or 2),
    list length, hot capacity, context range, growth a step and the pool's
    slack, which sets how soon evictions and new leases start."""
    rs = np.random.default_rng(4000 + seed)
    group = int(rs.choice([1, 2]))
    C = 64 * int(rs.integers(2, 17))
    return dict(name=f"policy_sweep_{seed}", seed=5000 + seed, R=int(rs.integers(2, 11)),
                L=group * int(rs.integers(1, 3)), K=int(rs.integers(16, 513)), C=C,
                steps=int(rs.integers(8, 21)), ctx_lo=int(rs.integers(1024, 6000)),
                ctx_hi=int(rs.integers(6000, 14000)), append=int(rs.integers(1, 80)),
                slack=int(rs.integers(4, 40)), tail_pages=int(rs.integers(1, 6)), group=group)


@pytest.mark.parametrize("seed", list(range(6)))
def test_policy_driven_sweep(seed):
    """Policy-driven runs of random shapes, every step against the oracle."""
    wl, dec = policy_workload(**_policy_sweep_params(seed))
    run_parity(wl)


def test_policy_driven_decode():
    """The same at decode size: 32 requests at 60-80 k tokens, top-K 2048,
    hot buffer 4096, 64 tokens appended per step."""
    wl, dec = policy_workload(name="policy_decode_32", seed=1007, R=32, L=1, K=2048, C=4096,
                              steps=10, ctx_lo=60000, ctx_hi=80000, append=64, slack=64,
                              tail_pages=16, n_host_blocks=2048)
    _say(f"[parity] policy decode: {dec.evicted} evictions, {dec.leased} leases")
    assert dec.evicted > 0
    totals = run_parity(wl)
    _say(f"[parity] policy_decode totals {totals.tolist()}")
    assert totals[2] > 0


def test_plan_rows_replayed_by_gather():
    """Speculative decoding ("Integration with the rest of vLLM": a per-step
    replayable plan): the draft and verify forwards of a step re-read the
    plan's rows with hs_gather on its row ids, at the hot buffer size for
    three speculative tokens, and get exactly the plan's own gathered rows."""
    from serving_memory_tier_amd.runner import DeviceRun
    wl = hs_gen.mtp_state(steps=3)
    dev = DeviceRun(wl)
    dev.upload_steps()
    try:
        for i in range(len(wl.steps)):
            _say(f"[parity] plan replay step {i}")
            dev.pre(i)
            dev.plan_step(i)
            torch.cuda.synchronize()
            planned = dev.out.clone()
            for forward in range(2):       # draft, then verify
                dev.out.zero_()
                dev.gather()
                torch.cuda.synchronize()
                assert torch.equal(dev.out, planned), f"forward {forward}, step {i}"
    finally:
        dev.close()


@pytest.mark.parametrize("R", [8, 48])
def test_concurrent_calls_on_two_streams(R):
    """Two batches with misses resolved by calls running at the same time on
    two streams (each with its own state, outputs and fill_sync counters):
    the misses' shared host reads of one call never mix with the other's,
    and both match the oracle bit for bit, every step.  With 48 requests the
    miss workgroups take their items from the counters."""
    from serving_memory_tier_amd.runner import DeviceRun

    wls = [hs_gen.mixed_decode(seed=1001 + k, steps=4, R=R) for k in range(2)]
    devs = [DeviceRun(wl) for wl in wls]
    oras = [OracleRun(wl) for wl in wls]
    streams = [torch.cuda.Stream() for _ in wls]
    try:
        for d in devs:
            d.upload_steps()
        for i in range(4):
            _say(f"[parity] two streams, step {i}")
            for d, o, wl in zip(devs, oras, wls):
                d.pre(i)
                o.pre(wl.steps[i])
            torch.cuda.synchronize()
            for d, s in zip(devs, streams):
                d.resolve(i, stream=s)
            torch.cuda.synchronize()
            for k, (d, o, wl) in enumerate(zip(devs, oras, wls)):
                rows, stats, out = o.resolve(wl.steps[i])
                assert int(stats[..., 2].sum()) > 0, "the step has misses"
                assert np.array_equal(d.rows.cpu().numpy(), rows), f"row ids, batch {k}"
                assert np.array_equal(d.stats.cpu().numpy(), stats), f"stats, batch {k}"
                assert np.array_equal(d.out.cpu().numpy(), out), f"gathered rows, batch {k}"
                assert np.array_equal(d.tok.cpu().numpy(), o.tok), f"slot tokens, batch {k}"
                assert np.array_equal(d.pool.cpu().numpy(), o.pool), f"pool, batch {k}"
    finally:
        for d in devs:
            d.close()


@pytest.mark.parametrize("make", ["mixed_state", "multi_layer", "in_place"])
def test_fill_sync_items(make):
    """More (request-layer, split) items than miss workgroups: with the
    batch's fill_sync each miss workgroup takes its next item from a counter,
    without it each takes a fixed share.  Both give identical row ids, stats,
    gathered bytes, state and pool, step after step and on the hit replay of
    each step, and every call leaves the counters zero.  ``in_place``: the
    misses-only fill with its staging rows (hs_resolve_in_place)."""
    from serving_memory_tier_amd.runner import DeviceRun

    wl = (hs_gen.mixed_state(R=48, steps=4) if make == "mixed_state"
          else hs_gen.multi_layer(R=4, L=16, turns=3) if make == "multi_layer"
          else hs_gen.mixed_decode(R=40, steps=4))
    a, b = DeviceRun(wl), DeviceRun(wl, fill_sync=False)
    assert a.fill_sync is not None and b.fill_sync is None
    mode = "in_place" if make == "in_place" else "call"
    misses = 0
    try:
        for d in (a, b):
            d.upload_steps()
        for i in range(len(wl.steps)):
            _say(f"[parity] fill_sync {make} step {i}")
            for d in (a, b):
                d.pre(i)
            for rep in range(2):  # the step, then its hit replay
                for d in (a, b):
                    if mode == "call":
                        d.resolve(i)
                    else:
                        stages.run(mode, d.layout, d.batch, d.topk[i], wl.P, wl.K,
                                   wl.steps[i].stamp, d.rows, d.out, d.stats)
                torch.cuda.synchronize()
                if rep == 0:
                    misses += int(a.stats[..., 2].sum())
                assert int(torch.count_nonzero(a.fill_sync)) == 0, f"counters, step {i}"
                pairs = [(a.rows, b.rows), (a.stats, b.stats), (a.tok, b.tok), (a.stp, b.stp),
                         (a.pool, b.pool)]
                if mode == "call":  # in place, the output holds staging rows only
                    pairs.append((a.out, b.out))
                for x, y in pairs:
                    assert torch.equal(x, y), f"step {i}, replay {rep}"
            for d in (a, b):
                d.post(i)
        torch.cuda.synchronize()
        assert torch.equal(a.host, b.host)
        assert misses > 0
    finally:
        a.close()
        b.close()
