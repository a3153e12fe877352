"""Shared test plumbing: running a synthetic workload through the CPU oracle,
building tiny hand-made instances, and checking gathered rows against the
content each token must hold."""

from __future__ import annotations

import numpy as np
import torch

import hs_gen
import oracle

ROW = hs_gen.ROW_BYTES
PAGE = hs_gen.PAGE


class OracleRun:
    """The full state of a workload on the CPU, advanced step by step by the oracle.

    With ``requests`` only those requests are simulated (request-layers are
    independent, so a subset resolves exactly as it does inside the batch):
    their pages are written to a full-size pool (the rest stays zero), and the
    tables, state, top-K lists and offload pairs are cut to the subset.
    """

    def __init__(self, wl: hs_gen.Workload, requests=None, content_device=None, threads=1):
        self.wl = wl
        self.threads = threads
        if requests is not None and wl.dynamic:
            raise ValueError("blocks move between requests: simulate the whole batch")
        self.req = np.arange(wl.R) if requests is None else np.asarray(requests, dtype=np.int64)
        R = self.req.size
        self.pool = np.zeros((wl.L, wl.pool_rows, ROW), dtype=np.uint8)
        self.host = np.zeros((wl.L, wl.host_rows, ROW), dtype=np.uint8)
        # the generator's rows, computed where the caller says (its torch and
        # numpy forms are pinned bit-identical)
        wl.fill_device_pool(torch.from_numpy(self.pool), compute_device=content_device,
                            requests=None if requests is None else self.req)
        wl.fill_host_pool(torch.from_numpy(self.host), compute_device=content_device)
        self.bt = np.ascontiguousarray(wl.block_table[self.req])
        self.hbt = np.ascontiguousarray(wl.host_block_table[self.req])
        self.hot = np.ascontiguousarray(wl.hot_blocks[self.req])
        self.ctx = np.ascontiguousarray(wl.ctx0[self.req])
        # hot-buffer state per layer group (one group per layer unless the
        # workload's layers share top-K lists)
        self.tok = np.full((R, wl.NG, wl.C), -1, dtype=np.int32)
        self.stp = np.zeros((R, wl.NG, wl.C), dtype=np.uint32)
        blocks = wl.dev_pages[np.isin(wl.dev_pages[:, 0], self.req), 2]
        self.own_blocks = set(blocks.tolist())
        self.pos = {int(r): i for i, r in enumerate(self.req)}

    def _rows_of(self, arr):
        keep = np.isin(arr[:, 0], self.req)
        a = arr[keep].copy()
        a[:, 0] = [self.pos[int(r)] for r in a[:, 0]]
        return a

    def pre(self, step: hs_gen.Step) -> None:
        for r, p, v in self._rows_of(step.hbt_set):
            self.hbt[r, p] = v
        for r, p, v in self._rows_of(step.bt_set):
            self.bt[r, p] = v
        for r, j, v in self._rows_of(step.hot_set):
            self.hot[r, j] = v
        for r in step.reset:
            if int(r) in self.pos:
                self.tok[self.pos[int(r)]] = -1
                self.stp[self.pos[int(r)]] = 0
        self.wl.write_pages(torch.from_numpy(self.pool), step.new_pages)
        self.ctx = np.ascontiguousarray(step.ctx[self.req])

    def resolve(self, step: hs_gen.Step, gather: bool = True, topk=None, stamp=None):
        topk = np.ascontiguousarray(step.topk[self.req] if topk is None else topk)
        stamp = step.stamp if stamp is None else stamp
        R = self.req.size
        if self.threads <= 1 or R < 2:
            return self._resolve_block(0, R, topk, stamp, gather)
        # request-layers are independent and their hot blocks disjoint, so
        # blocks of requests resolve on threads of their own (the oracle
        # releases the GIL); each block's state and lists are contiguous
        # slices of the batch's arrays
        from concurrent.futures import ThreadPoolExecutor
        n = min(self.threads, R)
        cuts = [R * i // n for i in range(n + 1)]
        with ThreadPoolExecutor(n) as ex:
            parts = list(ex.map(lambda i: self._resolve_block(cuts[i], cuts[i + 1], topk, stamp,
                                                              gather), range(n)))
        rows = np.concatenate([p[0] for p in parts])
        stats = np.concatenate([p[1] for p in parts])
        out = np.concatenate([p[2] for p in parts]) if gather else None
        return rows, stats, out

    def _resolve_block(self, r0, r1, topk, stamp, gather):
        a = [x[r0:r1] for x in (self.bt, self.hbt, self.ctx, self.hot, self.tok, self.stp, topk)]
        if self.wl.G > 1:
            return oracle.resolve_grouped(self.pool, self.host, *a, stamp, self.wl.G, gather)
        return oracle.resolve(self.pool, self.host, *a, stamp, gather)

    def pairs(self, step: hs_gen.Step) -> np.ndarray:
        if self.req.size == self.wl.R:
            return np.ascontiguousarray(step.offload).reshape(-1, 2)
        keep = [i for i, (db, _) in enumerate(step.offload) if int(db) in self.own_blocks]
        return np.ascontiguousarray(step.offload[keep]).reshape(-1, 2)

    def post(self, step: hs_gen.Step) -> None:
        pr = self.pairs(step)
        if pr.shape[0]:
            oracle.offload(self.pool, self.host, pr)


class PolicyDecider:
    """The residency policy (libhs_policy.so) as a workload's step-by-step
    decider: admission and per-step edits, with the policy's host blocks
    below the workload's reused-prefix host blocks."""

    def __init__(self, R, n_blocks, n_host_blocks, max_pages, C, tail_pages):
        from serving_memory_tier_amd import policy as pol
        self.p = pol.Policy(PAGE, n_blocks, n_host_blocks, R, max_pages, C // PAGE, tail_pages)
        self.evicted = 0
        self.leased = 0

    def admit(self, r, ctx, host_block_of_page, resident_prefix):
        e = self.p.admit(r, ctx, host_block_of_page, resident_prefix)
        self.leased += e.leased
        return e

    def step(self, stamp, reqs, ctx, topk):
        e = self.p.step(stamp, reqs, ctx, topk)
        self.evicted += e.evicted
        self.leased += e.leased
        return e


def policy_workload(name="policy_decode", seed=1006, R=8, L=2, K=256, C=512, steps=24,
                    ctx_lo=4096, ctx_hi=12288, append=40, slack=24, tail_pages=4, group=1,
                    n_host_blocks=4096):
    """A decode workload whose residency the policy decides step by step.
    Even requests start fully resident (their prefix also on host), odd ones
    host-only behind placeholders; the pool holds what admission needs plus
    ``slack`` blocks, so the appended tokens soon force evictions of the
    coldest pages and new hot leases.  Returns (workload, decider)."""
    rs = np.random.default_rng(seed)
    ctx0 = rs.integers(ctx_lo, ctx_hi, size=R)
    classes = np.where(np.arange(R) % 2 == 0, 0, 2).astype(np.int8)
    pages0 = (ctx0 + PAGE - 1) // PAGE
    need = 0
    for r in range(R):
        need += int(pages0[r]) if classes[r] == 0 else tail_pages + C // PAGE
    n_blocks = need + slack
    max_pages = int((ctx0.max() + steps * append + PAGE - 1) // PAGE)
    dec = PolicyDecider(R, n_blocks, n_host_blocks, max_pages, C, tail_pages)
    spec = hs_gen.Spec(name=name, seed=seed, R=R, L=L, K=K, C=C, steps=steps, ctx0=ctx0,
                       classes=classes, append=append, group=group)
    wl = hs_gen.build_dynamic(spec, dec, n_blocks, n_host_blocks)
    return wl, dec


def expected_content(wl: hs_gen.Workload, topk: np.ndarray, rows: np.ndarray,
                     requests=None) -> np.ndarray:
    """What every gathered row must hold, from the token alone: its synthetic
    content where a row was resolved (row id >= 0), zeros elsewhere.  With
    layer groups, topk and rows are per group and the result per layer."""
    if wl.G > 1:
        topk = np.repeat(topk, wl.G, axis=1)
        rows = np.repeat(rows, wl.G, axis=1)
    R, L = topk.shape[:2]
    t = topk.reshape(R, L, -1).astype(np.int64)
    lay = np.broadcast_to(np.arange(L)[None, :, None], t.shape)
    srcs = wl.src if requests is None else wl.src[np.asarray(requests)]
    src = np.broadcast_to(srcs[:, None, None], t.shape)
    exp = hs_gen.content_np(lay.ravel(), src.ravel(), t.ravel()).reshape(t.shape + (ROW,))
    ok = rows.reshape(R, L, -1) >= 0
    exp[~ok] = 0
    return exp.reshape(topk.shape + (ROW,))


def tiny_instance(page=4, ctx=24, C=8, hot_blocks=(9, 6), bt=(-1, -1, -1, -1, 7, 2),
                  hbt=(3, 0, 5, 1, 4, 2), n_blocks=10, n_host=6, seed=7):
    """The hand-worked instance: pool and host rows carry recognisable bytes
    (row r of layer 0 starts with r as little-endian int32, plus a tag byte)."""
    pool = np.zeros((1, n_blocks * page, ROW), dtype=np.uint8)
    host = np.zeros((1, n_host * page, ROW), dtype=np.uint8)
    for r in range(n_blocks * page):
        pool[0, r, :4] = np.frombuffer(np.int32(r).tobytes(), np.uint8)
        pool[0, r, 4] = 0xD0
    for r in range(n_host * page):
        host[0, r, :4] = np.frombuffer(np.int32(r).tobytes(), np.uint8)
        host[0, r, 4] = 0x40
    return dict(
        page=page, pool=pool, host=host,
        bt=np.array([bt], dtype=np.int32), hbt=np.array([hbt], dtype=np.int32),
        ctx=np.array([ctx], dtype=np.int32), hot=np.array([hot_blocks], dtype=np.int32),
        tok=np.full((1, 1, C), -1, dtype=np.int32), stp=np.zeros((1, 1, C), dtype=np.uint32))


def run_tiny(inst, topk, stamp, gather=True):
    t = np.asarray(topk, dtype=np.int32)
    t = t.reshape((1, 1) + t.shape) if t.ndim == 1 else t.reshape((1, 1) + t.shape)
    return oracle.resolve(inst["pool"], inst["host"], inst["bt"], inst["hbt"], inst["ctx"],
                          inst["hot"], inst["tok"], inst["stp"], t, stamp, gather,
                          page=inst["page"])
