"""Device-side driver for a workload: owns the GPU buffers of one batch (pool,
pinned host pool, tables, hot-buffer state) and steps it through the hot path.

Between steps it applies the scheduler's decisions the workload describes --
nulling pages that left the resident tail, recording new host copies, and
for workloads whose residency policy runs step by step new pool blocks with
their rows, hot-block leases and the reset of a re-leased hot buffer -- as
plain device-tensor writes; these are host-side residency policy, not part of
the hot path.  Each step then calls the C ABI through the binding:
``hs_resolve`` (or ``hs_plan_replay`` for several query positions), whose
gather runs on the same stream, and ``hs_offload_prefix_pages`` for the pages
that completed: in the launched steps on a second stream beside the resolve,
joined before the step ends.
"""

from __future__ import annotations

import numpy as np
import torch

from ._lib import HS_FILL_SYNC_WORDS
from .api import (HostPool, batch_of, hs_gather, hs_offload_prefix_pages, hs_plan_replay,
                  hs_resolve, hs_resolve_commit, hs_resolve_decide, hs_resolve_grouped,
                  hs_resolve_move, layout_of)

PAGE = 64
ROW = 656


def update_runs(arr: np.ndarray):
    """A step's table updates (rows of (request, page, value), one per entry) as
    runs that one copy each can write: whichever of two cuts gives fewer runs --
    columns (the same page of consecutive requests, max_pages entries apart: a
    completed page updates every request's entry at once) or rows (consecutive
    pages of one request, contiguous).  Yields (request, page, along_pages,
    int32 values) for the run starting at (request, page)."""
    if arr.shape[0] == 0:
        return []
    assert np.unique(arr[:, :2], axis=0).shape[0] == arr.shape[0], "one update per table entry"
    cuts = []
    for major, minor in ((1, 0), (0, 1)):   # columns, then rows
        a = arr[np.lexsort((arr[:, minor], arr[:, major]))]
        runs = []
        j = 0
        while j < a.shape[0]:
            e = j + 1
            while (e < a.shape[0] and a[e, major] == a[j, major]
                   and a[e, minor] == a[e - 1, minor] + 1):
                e += 1
            runs.append((int(a[j, 0]), int(a[j, 1]), minor == 1, a[j:e, 2].astype(np.int32)))
            j = e
        cuts.append(runs)
    return min(cuts, key=len)


# offloads from this size up run beside the resolve (launch_step): the
# multi-layer turn's 505 MB, not a decode step's few pages
OVERLAP_BYTES = 64 << 20


class DeviceRun:
    def __init__(self, wl, device: str = "cuda", content_device: str | None = None,
                 fill_sync: bool = True):
        self.wl = wl
        dev = torch.device(device)
        self.device = dev
        cdev = content_device or device
        self.cdev = cdev
        self.pool = torch.zeros((wl.L, wl.pool_rows, ROW), dtype=torch.uint8, device=dev)
        wl.fill_device_pool(self.pool, compute_device=cdev)
        self.host_pool = HostPool(wl.L * wl.host_rows * ROW)
        self.host = self.host_pool.tensor.view(wl.L, wl.host_rows, ROW)
        self.host.zero_()
        wl.fill_host_pool(self.host, compute_device=cdev)
        i32 = torch.int32
        self.bt = torch.from_numpy(wl.block_table).to(dev)
        self.hbt = torch.from_numpy(wl.host_block_table).to(dev)
        self.ctx = torch.from_numpy(wl.ctx0.astype(np.int32)).to(dev)
        self.hot = torch.from_numpy(wl.hot_blocks).to(dev)
        # hot-buffer state, lists, row ids and stats per layer group (one group
        # per layer unless the workload's layers share top-K lists); the
        # output has every layer's rows
        NG = wl.NG
        self.tok = torch.full((wl.R, NG, wl.C), -1, dtype=i32, device=dev)
        self.stp = torch.zeros((wl.R, NG, wl.C), dtype=i32, device=dev)  # uint32 bits
        N = wl.P * wl.K
        self.rows = torch.empty((wl.R, NG, wl.P, wl.K), dtype=i32, device=dev)
        self.stats = torch.empty((wl.R, NG, 8), dtype=i32, device=dev)
        self.out = torch.empty((wl.R, wl.L, wl.P, wl.K, ROW), dtype=torch.uint8, device=dev)
        self.layout = layout_of(PAGE, ROW, wl.L, wl.C, wl.pool_rows, wl.host_rows)
        # the miss workgroups' item counters (zero between calls)
        self.fill_sync = (torch.zeros(HS_FILL_SYNC_WORDS, dtype=i32, device=dev)
                          if fill_sync else None)
        self.batch = batch_of(wl.R, wl.max_pages, self.pool, self.host_pool, self.bt, self.hbt,
                              self.ctx, self.hot, self.tok, self.stp, self.fill_sync)
        self.entries = N
        self.topk = [None] * len(wl.steps)
        self.pairs = [None] * len(wl.steps)
        # a step's prefix-page offload runs on a second stream, beside its
        # resolve (device -> host against the resolve's host -> device reads);
        # default priority, forked and joined by events inside the step
        self.side = torch.cuda.Stream(device=dev)

    # -- scheduler side (between steps) ------------------------------------
    def upload_steps(self) -> None:
        """Put every step's top-K lists and offload pairs in device memory."""
        for i, s in enumerate(self.wl.steps):
            self.topk[i] = torch.from_numpy(np.ascontiguousarray(s.topk)).to(self.device)
            self.pairs[i] = (torch.from_numpy(np.ascontiguousarray(s.offload)).to(self.device)
                             if s.offload.shape[0] else None)

    def pre(self, i: int) -> None:
        s = self.wl.steps[i]
        for arr, t in ((s.hbt_set, self.hbt), (s.bt_set, self.bt), (s.hot_set, self.hot)):
            if arr.shape[0]:
                a = torch.from_numpy(arr).to(self.device)
                t[a[:, 0], a[:, 1]] = a[:, 2].to(torch.int32)
        if s.reset.shape[0]:
            # a new or returned lease: the request's hot buffer starts empty
            rr = torch.from_numpy(s.reset).to(self.device)
            self.tok[rr] = -1
            self.stp[rr] = 0
        # pages that took a block (possibly one another page or lease held)
        # get their rows, as the forward pass writes them
        self.wl.write_pages(self.pool, s.new_pages, compute_device=self.cdev)
        self.ctx.copy_(torch.from_numpy(s.ctx.astype(np.int32)))

    # -- hot path -----------------------------------------------------------
    def resolve(self, i: int, gather: bool = True, stamp: int | None = None, topk=None,
                stream=None) -> None:
        s = self.wl.steps[i]
        if topk is None:
            if self.topk[i] is None:
                self.topk[i] = torch.from_numpy(np.ascontiguousarray(s.topk)).to(self.device)
            topk = self.topk[i]
        stamp = s.stamp if stamp is None else stamp
        out = self.out if gather else None
        if self.wl.G > 1:
            hs_resolve_grouped(self.layout, self.batch, self.wl.G, topk, self.wl.P, self.wl.K,
                               stamp, self.rows, out, self.stats, None, 0, stream)
        elif self.wl.P == 1:
            hs_resolve(self.layout, self.batch, topk, self.wl.K, stamp, self.rows, out,
                       self.stats, stream)
        else:
            hs_plan_replay(self.layout, self.batch, topk, self.wl.P, self.wl.K, stamp, self.rows,
                           out, self.stats, None, 0, stream)

    def gather(self, stream=None) -> None:
        assert self.wl.G == 1, "row ids are per layer group; gather each layer's plane"
        hs_gather(self.layout, self.pool, self.rows, self.wl.R, self.entries, self.out, stream)

    def post(self, i: int, stream=None) -> None:
        s = self.wl.steps[i]
        if s.offload.shape[0] == 0:
            return
        if self.pairs[i] is None:
            self.pairs[i] = torch.from_numpy(np.ascontiguousarray(s.offload)).to(self.device)
        hs_offload_prefix_pages(self.layout, self.pool, self.host_pool, self.pairs[i],
                                s.offload.shape[0], stream)

    def plan_step(self, i: int, gather: bool = True, stream=None) -> None:
        """resolve + gather + offload of the step's completed pages, one call."""
        s = self.wl.steps[i]
        if self.topk[i] is None:
            self.topk[i] = torch.from_numpy(np.ascontiguousarray(s.topk)).to(self.device)
        n = s.offload.shape[0]
        if n and self.pairs[i] is None:
            self.pairs[i] = torch.from_numpy(np.ascontiguousarray(s.offload)).to(self.device)
        if self.wl.G > 1:
            hs_resolve_grouped(self.layout, self.batch, self.wl.G, self.topk[i], self.wl.P,
                               self.wl.K, s.stamp, self.rows, self.out if gather else None,
                               self.stats, self.pairs[i] if n else None, n, stream)
            return
        hs_plan_replay(self.layout, self.batch, self.topk[i], self.wl.P, self.wl.K, s.stamp,
                       self.rows, self.out if gather else None, self.stats,
                       self.pairs[i] if n else None, n, stream)

    # -- steps with no host work between them ----------------------------------
    def stage_steps(self) -> None:
        """Stage every step's context lengths and table updates in device and
        pinned memory, so that a run of steps (``launch_step``) needs no host
        work between kernels and captures into a graph as it stands."""
        wl = self.wl
        if wl.dynamic:
            raise ValueError("steps with lease changes and page writes need pre() between them")
        n = len(wl.steps)
        self.ctx_all = torch.from_numpy(
            np.stack([s.ctx for s in wl.steps]).astype(np.int32)).to(self.device)
        self.batches = [batch_of(wl.R, wl.max_pages, self.pool, self.host_pool, self.bt,
                                 self.hbt, self.ctx_all[i], self.hot, self.tok, self.stp,
                                 self.fill_sync)
                        for i in range(n)]
        n_vals = sum(s.hbt_set.shape[0] + s.bt_set.shape[0] for s in wl.steps)
        self.pinned_vals = torch.empty(max(1, n_vals), dtype=torch.int32, pin_memory=True)
        # each step's updates as copies of runs (update_runs), one copy a run
        self.table_sets = []
        k = 0
        for s in wl.steps:
            sets = []
            for arr, t in ((s.hbt_set, self.hbt), (s.bt_set, self.bt)):
                for r, p, along_pages, vals in update_runs(arr):
                    n_run = vals.shape[0]
                    self.pinned_vals[k:k + n_run] = torch.from_numpy(vals)
                    pitch = 4 if along_pages else 4 * wl.max_pages
                    sets.append((t.data_ptr() + 4 * (r * wl.max_pages + p), pitch,
                                 self.pinned_vals.data_ptr() + 4 * k, n_run))
                    k += n_run
            self.table_sets.append(sets)

    def _table_updates(self, i: int, hip, stream: int) -> None:
        for dst, pitch, src, n in self.table_sets[i]:
            if n == 1 or pitch == 4:
                hip.memcpy_h2d(dst, src, 4 * n, stream)
            else:
                hip.memcpy2d_h2d(dst, pitch, src, 4, 4, n, stream)

    def launch_step(self, i: int, hip, stream: int, stats=None, serial: bool = False,
                    offload: bool = True, overlap: bool = True) -> None:
        """Step ``i`` on ``stream`` with no host work: the scheduler's table
        updates as copies from pinned memory, then the resolve (one
        hs_plan_replay call: fused resolve and gather, commit) and the offload
        of the pages the step completed.
        ``overlap``: an offload of at least OVERLAP_BYTES runs on a second
        stream beside the resolve, forked after the table updates and joined
        before the step ends (the link carries the offload's writes to host
        and the misses' reads from it at once; the offloaded pages are
        resident, so the resolve reads them in place, never their host copies
        being written).  Smaller offloads, or False: one hs_plan_replay call
        with the offload pairs, the offload after the commit on ``stream``
        (the fork and join cost more than a short offload gives back).
        ``serial``: the decide and move stages one after the other instead
        (the path the library takes without a gather output, with one).
        ``offload``: False leaves out the step's prefix-page offload."""
        wl = self.wl
        s = wl.steps[i]
        self._table_updates(i, hip, stream)
        st = self.stats if stats is None else stats
        n_off = s.offload.shape[0] if offload else 0
        join = None
        if n_off and overlap and not serial and n_off * wl.L * PAGE * ROW >= OVERLAP_BYTES:
            fork, join = hip.new_event(), hip.new_event()  # owned by `hip`
            side = self.side.cuda_stream
            hip.record(fork, stream)
            hip.wait(side, fork)
            hs_offload_prefix_pages(self.layout, self.pool, self.host_pool, self.pairs[i], n_off,
                                    side)
            hip.record(join, side)
            n_off = 0  # the resolve below carries no offload
        if wl.G > 1:
            assert not serial, "layer groups have no serial staged form"
            hs_resolve_grouped(self.layout, self.batches[i], wl.G, self.topk[i], wl.P, wl.K,
                               s.stamp, self.rows, self.out, st,
                               self.pairs[i] if n_off else None, n_off, stream)
        elif serial:
            hs_resolve_decide(self.layout, self.batches[i], self.topk[i], wl.P, wl.K, s.stamp,
                              self.rows, None, st, stream)
            hs_resolve_move(self.layout, self.batches[i], self.topk[i], wl.P, wl.K, self.rows,
                            self.out, stream)
            if n_off:
                hs_offload_prefix_pages(self.layout, self.pool, self.host_pool, self.pairs[i],
                                        n_off, stream)
        else:
            hs_plan_replay(self.layout, self.batches[i], self.topk[i], wl.P, wl.K, s.stamp,
                           self.rows, self.out, st, self.pairs[i] if n_off else None, n_off,
                           stream)
        if join is not None:
            hip.wait(stream, join)

    def launch_step_timed(self, i: int, hip, stream: int, ev, stats=None,
                          offload: bool = True) -> None:
        """Step ``i`` as the stages of hs_plan_replay on ``stream`` -- the fused
        resolve-and-fill launch, the commit, the offload -- with events around
        each kernel: ``ev`` holds four events, recorded before the fused
        launch, after it, after the commit and after the offload."""
        wl = self.wl
        s = wl.steps[i]
        self._table_updates(i, hip, stream)
        st = self.stats if stats is None else stats
        L, B, T = self.layout, self.batches[i], self.topk[i]
        if wl.G > 1:
            # one call: its fused launch, commit and offload under one event pair
            n_off = s.offload.shape[0] if offload else 0
            hip.record(ev[0], stream)
            hs_resolve_grouped(L, B, wl.G, T, wl.P, wl.K, s.stamp, self.rows, self.out, st,
                               self.pairs[i] if n_off else None, n_off, stream)
            for k in (1, 2, 3):
                hip.record(ev[k], stream)
            return
        hip.record(ev[0], stream)
        hs_resolve_decide(L, B, T, wl.P, wl.K, s.stamp, self.rows, self.out, st, stream)
        hip.record(ev[1], stream)
        hs_resolve_commit(L, B, T, wl.P, wl.K, self.rows, self.out, stream)
        hip.record(ev[2], stream)
        n_off = s.offload.shape[0] if offload else 0
        if n_off:
            hs_offload_prefix_pages(L, self.pool, self.host_pool, self.pairs[i], n_off, stream)
        hip.record(ev[3], stream)

    def close(self) -> None:
        self.host = None
        self.host_pool.close()
