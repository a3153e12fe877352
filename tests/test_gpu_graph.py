"""A captured HIP graph of the hot path gives the eager results on every replay.

Several decode steps (the scheduler's table updates as 4-byte copies from
pinned memory, the decide and move kernels, the prefix offload) are captured
once into a graph and replayed three times from the same starting state.
Between replays the program does eager work of its own (restoring the state,
poisoning the outputs, an unrelated matmul and reduction) and synchronises.
Every replay must reproduce, byte for byte, what the same steps give when
launched eagerly on a second copy of the batch: row ids, stats and gathered
rows of every step, and the hot-buffer state, device pool and host pool at
the end.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import hs_gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    import serving_memory_tier_amd as hs
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hs.lib()


class _Recorder:
    """Per-step copies of a run's outputs, made on the launch stream."""

    def __init__(self, dev, n):
        self.rows = torch.empty((n,) + tuple(dev.rows.shape), dtype=dev.rows.dtype,
                                device=dev.rows.device)
        self.out = torch.empty((n,) + tuple(dev.out.shape), dtype=dev.out.dtype,
                               device=dev.out.device)
        self.stats = torch.empty((n,) + tuple(dev.stats.shape), dtype=dev.stats.dtype,
                                 device=dev.stats.device)

    def take(self, j, dev):
        self.rows[j].copy_(dev.rows)
        self.out[j].copy_(dev.out)

    def poison(self):
        self.rows.fill_(-5)
        self.out.fill_(0xEE)
        self.stats.fill_(-7)


def _snapshot(dev):
    torch.cuda.synchronize()
    return {"tok": dev.tok.clone(), "stp": dev.stp.clone(), "pool": dev.pool.clone(),
            "bt": dev.bt.clone(), "hbt": dev.hbt.clone(), "host": dev.host.numpy().copy()}


def _restore(dev, snap):
    torch.cuda.synchronize()
    dev.host.numpy()[...] = snap["host"]
    for k in ("tok", "stp", "pool", "bt", "hbt"):
        getattr(dev, k).copy_(snap[k])


@pytest.mark.parametrize("wl_name", ["mixed_decode", "multi_layer", "multi_layer_wide"])
def test_graph_replays_match_eager(wl_name):
    from serving_memory_tier_amd.hipgraph import HipRuntime
    from serving_memory_tier_amd.runner import DeviceRun

    if wl_name == "mixed_decode":
        # the captured steps include step 16, where a page completes and every
        # request's host-table entry for it is set (one strided copy)
        wl = hs_gen.mixed_decode(R=8, steps=20)
        warm, n_cap = 12, 6
        assert wl.steps[16].hbt_set.shape[0] == 8
    elif wl_name == "multi_layer":
        # turns with prefill, completed pages offloaded and pages leaving the tail
        wl = hs_gen.multi_layer(turns=4, R=4, L=4)
        warm, n_cap = 1, 3
        assert sum(s.offload.shape[0] + s.bt_set.shape[0] for s in wl.steps[1:]) > 0
    else:
        # 160 request-layers: more than half a round of resolver workgroups, so
        # the captured fused launches interleave resolvers and gathers
        wl = hs_gen.multi_layer(turns=3, R=40, L=4)
        warm, n_cap = 1, 2
    hip = HipRuntime()
    runs = [DeviceRun(wl), DeviceRun(wl)]
    eager, graphed = runs
    try:
        for d in runs:
            d.upload_steps()
            d.stage_steps()
        sp = torch.cuda.current_stream().cuda_stream
        for d in runs:
            for i in range(warm):
                d.launch_step(i, hip, sp)
        torch.cuda.synchronize()
        print(f"[graph] {wl_name}: warm {warm} steps, capturing {n_cap}", flush=True)

        # eager reference
        ref = _Recorder(eager, n_cap)
        for j in range(n_cap):
            eager.launch_step(warm + j, hip, sp, stats=ref.stats[j])
            ref.take(j, eager)
        torch.cuda.synchronize()
        ref_end = _snapshot(eager)
        # the staged table updates leave the tables the workload prescribes
        bt, hbt = wl.block_table.copy(), wl.host_block_table.copy()
        for s in wl.steps[:warm + n_cap]:
            for arr, t in ((s.hbt_set, hbt), (s.bt_set, bt)):
                for r, p, v in arr:
                    t[r, p] = v
        assert np.array_equal(ref_end["bt"].cpu().numpy(), bt), "block table after the updates"
        assert np.array_equal(ref_end["hbt"].cpu().numpy(), hbt), "host table after the updates"

        # capture the same steps on the second batch
        start = _snapshot(graphed)
        rec = _Recorder(graphed, n_cap)
        cap = torch.cuda.Stream()
        hip.begin_capture(cap.cuda_stream)
        try:
            with torch.cuda.stream(cap):
                for j in range(n_cap):
                    graphed.launch_step(warm + j, hip, cap.cuda_stream, stats=rec.stats[j])
                    rec.take(j, graphed)
        finally:
            hip.end_capture(cap.cuda_stream)

        a = torch.randn(512, 512, device="cuda")
        for replay in range(3):
            _restore(graphed, start)
            rec.poison()
            graphed.out.fill_(0x11)
            graphed.rows.fill_(-3)
            _ = float((a @ a).sum())          # unrelated eager work
            torch.cuda.synchronize()
            hip.launch(cap.cuda_stream)
            torch.cuda.synchronize()
            print(f"[graph] {wl_name}: replay {replay} done", flush=True)
            for j in range(n_cap):
                assert torch.equal(rec.rows[j], ref.rows[j]), f"rows, replay {replay} step {j}"
                assert torch.equal(rec.stats[j], ref.stats[j]), f"stats, replay {replay} step {j}"
                assert torch.equal(rec.out[j], ref.out[j]), f"gather, replay {replay} step {j}"
            end = _snapshot(graphed)
            for k in ("tok", "stp", "pool", "bt", "hbt"):
                assert torch.equal(end[k], ref_end[k]), f"{k} after replay {replay}"
            assert np.array_equal(end["host"], ref_end["host"]), f"host pool, replay {replay}"
        s = ref.stats.sum(dim=(0, 1, 2)).cpu().numpy()
        assert s[2] > 0 and s[1] > 0, "the captured steps must both copy and hit"
    finally:
        hip.close()
        for d in runs:
            d.close()


@pytest.mark.parametrize("wl_name", ["mixed_decode", "multi_layer"])
def test_offload_beside_the_resolve_matches_in_order(wl_name):
    """A step whose offload runs on a second stream beside the resolve (the
    runner's default) leaves every byte -- rows, stats, gathered rows, state,
    both pools -- as the same step with the offload after the commit on one
    stream, step after step."""
    from serving_memory_tier_amd.hipgraph import HipRuntime
    from serving_memory_tier_amd.runner import DeviceRun

    if wl_name == "mixed_decode":
        wl = hs_gen.mixed_decode(R=8, steps=20)
        steps = range(12, 20)                     # step 16 offloads a completed page
    else:
        wl = hs_gen.multi_layer(turns=4, R=4, L=4)
        steps = range(4)
    assert sum(wl.steps[i].offload.shape[0] for i in steps) > 0
    import serving_memory_tier_amd.runner as runner
    hip = HipRuntime()
    a, b = DeviceRun(wl), DeviceRun(wl)
    saved = runner.OVERLAP_BYTES
    runner.OVERLAP_BYTES = 0          # every offload beside the resolve in `a`
    try:
        for d in (a, b):
            d.upload_steps()
            d.stage_steps()
        sp = torch.cuda.current_stream().cuda_stream
        for d in (a, b):
            for i in range(steps[0]):
                d.launch_step(i, hip, sp, overlap=False)
        torch.cuda.synchronize()
        for i in steps:
            print(f"[graph] {wl_name}: offload beside the resolve, step {i}", flush=True)
            a.launch_step(i, hip, sp, overlap=True)
            b.launch_step(i, hip, sp, overlap=False)
            torch.cuda.synchronize()
            for x, y in ((a.rows, b.rows), (a.stats, b.stats), (a.out, b.out), (a.tok, b.tok),
                         (a.stp, b.stp), (a.pool, b.pool), (a.bt, b.bt), (a.hbt, b.hbt)):
                assert torch.equal(x, y), f"step {i}"
            assert np.array_equal(a.host.numpy(), b.host.numpy()), f"host pool, step {i}"
    finally:
        runner.OVERLAP_BYTES = saved
        a.close()
        b.close()
        hip.close()

