"""Seeded synthetic workloads for the top-K resolver, gather and prefix offload.

This module only builds *inputs*: contexts, block tables (real blocks and
null placeholders), host block tables, hot-buffer block leases, the indexer's
top-K lists per step and the list of completed prefix pages to copy to host
after each step.  It never resolves a token, never touches hot-buffer state
and never computes a row id.  It serves the CPU oracle and the GPU path alike.

Workload shapes follow the pages' description of the problem ("vLLM GLM 5.3
... Hybrid HiSparse offloading, Part 1"):

* page-granular residency with three request states -- full, mixed (a GPU
  tail that never leaves, older pages host-only behind null placeholders) and
  none (a host-only prefix, placeholders plus a real page for new tokens)
  ("How it works", the three residency states);
* a hot buffer of 2 x top-K rows per request leased from the same block pool
  ("Integration with the rest of vLLM", hot-buffer default);
* completed prefix pages copied to host proactively ("How it works", the
  proactive copy), so every completed page starts with a host copy;
* the OpenHands multi-turn agentic shape -- a 74,160-token first turn and
  753-token later turns, 13 turns, 142,000-token admission ("Validation with
  numbers") -- stands in for the dataset the pages benchmark on.

Conventions: null block-table entry = -1, "no host copy" = -1, tokens of a
request are 0..ctx-1, page p holds tokens 64p..64p+63, stamps are step+1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import rng
from .content import PAGE, ROW_BYTES, fill_rows


@dataclass
class Step:
    stamp: int
    ctx: np.ndarray            # int32 [R], context length during this step
    topk: np.ndarray           # int32 [R, L // G, P, K]: one list per layer group
    bt_set: np.ndarray         # int64 [n, 3] (r, page, value) applied before the step
    hbt_set: np.ndarray        # int64 [n, 3] (r, page, value) applied before the step
    offload: np.ndarray        # int32 [n, 2] (device block, host block) copied after the step
    # residency decided step by step (build_dynamic); empty for scripted workloads
    hot_set: np.ndarray = field(default_factory=lambda: np.zeros((0, 3), np.int64))
    reset: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    # pages that take a fresh pool block before the step: their rows (the
    # tokens of the page) are written into the block, as the forward would
    new_pages: np.ndarray = field(default_factory=lambda: np.zeros((0, 3), np.int64))


@dataclass
class Workload:
    name: str
    seed: int
    R: int
    L: int
    P: int
    K: int
    C: int
    n_blocks: int
    n_host_blocks: int
    max_pages: int
    ctx0: np.ndarray                # int32 [R]
    block_table: np.ndarray         # int32 [R, max_pages]  (initial)
    host_block_table: np.ndarray    # int32 [R, max_pages]  (initial)
    hot_blocks: np.ndarray          # int32 [R, C // 64]
    src: np.ndarray                 # int64 [R] content source of each request
    dev_pages: np.ndarray           # int64 [n, 3] (r, page, block) every page ever resident
    host_pages: np.ndarray          # int64 [n, 2] (host block, token base) initial host copies
    host_src: np.ndarray            # int64 [n] content source of each initial host page
    steps: list = field(default_factory=list)
    classes: np.ndarray | None = None   # int8 [R]: 0 full, 1 mixed, 2 none (informational)
    G: int = 1                          # layers per group sharing one top-K list (IndexShare)

    @property
    def dynamic(self) -> bool:
        """Residency decided step by step: blocks are reused and leases move."""
        return any(s.new_pages.shape[0] or s.hot_set.shape[0] or s.reset.shape[0]
                   for s in self.steps)

    @property
    def NG(self) -> int:
        """Layer groups: top-K lists and hot-buffer states per request."""
        return self.L // self.G

    @property
    def page(self) -> int:
        return PAGE

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES

    @property
    def pool_rows(self) -> int:
        return self.n_blocks * PAGE

    @property
    def host_rows(self) -> int:
        return self.n_host_blocks * PAGE

    @property
    def entries_per_step(self) -> int:
        return self.R * self.L * self.P * self.K

    # -- content -----------------------------------------------------------
    def fill_device_pool(self, pool: torch.Tensor, compute_device=None, requests=None) -> None:
        """Write every resident page's rows into ``pool`` (uint8 [L, rows, 656]).

        Hot blocks and unused blocks are left as they are (callers pass a
        zeroed pool).  Pages that become resident later in the run are written
        up front; their tokens stay invalid until the context reaches them.
        ``requests`` limits the fill to the pages of those requests.
        """
        dp = self.dev_pages
        if requests is not None:
            dp = dp[np.isin(dp[:, 0], np.asarray(requests))]
        self.write_pages(pool, dp, compute_device)

    def write_pages(self, pool: torch.Tensor, pages: np.ndarray, compute_device=None) -> None:
        """Write the rows of the pages (r, page, block) into their pool blocks
        (uint8 [L, rows, 656]), every layer: the tokens of the page, valid or
        not yet, as the forward pass would write them."""
        dp = np.asarray(pages, dtype=np.int64).reshape(-1, 3)
        if dp.shape[0] == 0:
            return
        r, p, b = dp[:, 0], dp[:, 1], dp[:, 2]
        o = np.arange(PAGE, dtype=np.int64)
        rows = torch.from_numpy((b[:, None] * PAGE + o[None, :]).ravel())
        toks = torch.from_numpy((p[:, None] * PAGE + o[None, :]).ravel())
        srcs = torch.from_numpy(np.repeat(self.src[r], PAGE))
        for layer in range(self.L):
            fill_rows(pool[layer], rows, layer, srcs, toks, compute_device=compute_device)

    def fill_host_pool(self, host: torch.Tensor, compute_device=None) -> None:
        """Write the initial host copies into ``host`` (uint8 [L, host_rows, 656])."""
        hb, base = self.host_pages[:, 0], self.host_pages[:, 1]
        o = np.arange(PAGE, dtype=np.int64)
        rows = torch.from_numpy((hb[:, None] * PAGE + o[None, :]).ravel())
        toks = torch.from_numpy((base[:, None] * PAGE + o[None, :]).ravel())
        srcs = torch.from_numpy(np.repeat(self.host_src, PAGE))
        for layer in range(self.L):
            fill_rows(host[layer], rows, layer, srcs, toks, compute_device=compute_device)


# ---------------------------------------------------------------------------
# top-K list construction

def _distinct(k: int, n: int, lo: int, hi: int, exclude: np.ndarray) -> np.ndarray:
    """``n`` distinct tokens in [lo, hi) not in ``exclude``, in draw order."""
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    avail = (hi - lo) - np.count_nonzero((exclude >= lo) & (exclude < hi))
    if avail < n:
        raise ValueError(f"cannot draw {n} distinct tokens from [{lo},{hi})")
    out = np.zeros(0, dtype=np.int64)
    ctr = 0
    while out.size < n:
        want = 2 * (n - out.size) + 64
        cand = rng.uniform_ints(k, ctr, want, lo, hi)
        ctr += want
        cand = np.concatenate([out, cand])
        _, first = np.unique(cand, return_index=True)
        cand = cand[np.sort(first)]
        cand = cand[~np.isin(cand, exclude)]
        out = cand[:n]
    return out


def _sample(k: int, pool: np.ndarray, n: int) -> np.ndarray:
    """``n`` elements of ``pool`` without replacement (seeded)."""
    if n > pool.size:
        raise ValueError("sample larger than population")
    return pool[rng.permutation(k, pool.size)[:n]]


def _shuffle(k: int, a: np.ndarray) -> np.ndarray:
    return a[rng.permutation(k, a.size)]


def _mix(k: int, prev: np.ndarray | None, ctx: int, K: int, overlap: int, recent: int,
         recent_window: int, first_recent_share: float) -> np.ndarray:
    """One top-K list: ``overlap`` tokens of ``prev``, ``recent`` from the last
    ``recent_window`` tokens, the rest uniform over the context; all distinct.
    Without a previous list the overlap share is drawn recent:uniform by
    ``first_recent_share``."""
    if prev is None:
        extra_recent = int(math.floor(overlap * first_recent_share))
        recent, overlap = recent + extra_recent, 0
    uniform = K - overlap - recent
    parts = []
    ov = _sample(rng.key(k, 1), prev, overlap) if overlap else np.zeros(0, np.int64)
    parts.append(ov)
    lo = max(0, ctx - recent_window)
    rc = _distinct(rng.key(k, 2), recent, lo, ctx, ov)
    un = _distinct(rng.key(k, 3), uniform, 0, ctx, np.concatenate([ov, rc]))
    return _shuffle(rng.key(k, 4), np.concatenate([ov, rc, un]))


def _split_counts(K: int, fractions: tuple) -> list:
    """Floor each named fraction of K; the remainder goes to the last class."""
    counts = [int(math.floor(f * K)) for f in fractions[:-1]]
    return counts + [K - sum(counts)]


# ---------------------------------------------------------------------------
# generic builder

@dataclass
class Spec:
    name: str
    seed: int
    R: int
    L: int
    K: int
    C: int
    steps: int
    ctx0: np.ndarray                 # int64 [R]
    classes: np.ndarray              # int8 [R]: 0 full, 1 mixed, 2 none
    tail_frac: float = 0.25          # resident tail of "mixed" requests (numerator/denominator via float)
    P: int = 1
    append: int = 1                  # tokens appended per step
    append_first: bool = True        # step 0 already appended `append` tokens
    mix: tuple = (0.70, 0.20, 0.10)  # overlap, recent, uniform
    recent_window: int = 4096
    first_recent_share: float = 2.0 / 3.0
    pos_keep: int = 1536             # positions 1.. : tokens kept from position 0
    shared_src: bool = False         # all requests read one source sequence (shared host pages)
    move_tail: bool = False          # null pages that leave the tail as the context grows
    group: int = 1                   # layers per group sharing one top-K list (IndexShare)


def _tail_first_page(ctx: int, frac: float) -> int:
    tail = int(math.ceil(frac * ctx - 1e-9))
    return max(0, (ctx - tail) // PAGE)


def build(spec: Spec) -> Workload:
    R, L, P, K, C = spec.R, spec.L, spec.P, spec.K, spec.C
    if C % PAGE:
        raise ValueError("hot capacity must be a whole number of pages")
    G = spec.group
    if G < 1 or L % G:
        raise ValueError("the layer group must divide the layers")
    NG = L // G
    seed = spec.seed
    ctx0 = spec.ctx0.astype(np.int64)
    d = 1 if spec.append_first else 0
    ctx_steps = [ctx0 + (s + d) * spec.append for s in range(spec.steps)]
    ctx_final = ctx_steps[-1] if spec.steps else ctx0
    max_pages = int(max(((ctx_final + PAGE - 1) // PAGE).max(), ((ctx0 + PAGE - 1) // PAGE).max()))

    # first resident page of each request at each step (and initially)
    def first_res(ctx_vec):
        out = np.zeros(R, dtype=np.int64)
        for r in range(R):
            c = int(ctx_vec[r])
            if spec.classes[r] == 0:
                out[r] = 0
            elif spec.classes[r] == 1:
                out[r] = _tail_first_page(c, spec.tail_frac)
            else:
                out[r] = int(ctx0[r]) // PAGE
        return out

    fr0 = first_res(ctx0)
    if spec.move_tail:
        fr_steps = [np.maximum(first_res(c), fr0) for c in ctx_steps]
    else:
        fr_steps = [fr0 for _ in ctx_steps]
    last_page = (ctx_final - 1) // PAGE   # last page any step touches

    # device blocks: every page that is resident at any point, then hot blocks
    n_res = [int(last_page[r] - fr0[r] + 1) for r in range(R)]
    n_hot = C // PAGE
    n_blocks = sum(n_res) + R * n_hot
    perm = rng.permutation(rng.key(seed, 0xB10C), n_blocks).astype(np.int64)
    bt = np.full((R, max_pages), -1, dtype=np.int32)
    hot = np.zeros((R, n_hot), dtype=np.int32)
    dev_pages = []
    cur = 0
    for r in range(R):
        pages = np.arange(fr0[r], last_page[r] + 1, dtype=np.int64)
        blocks = perm[cur:cur + pages.size]
        cur += pages.size
        bt[r, pages] = blocks
        dev_pages.append(np.stack([np.full(pages.size, r), pages, blocks], 1))
    for r in range(R):
        hot[r] = perm[cur:cur + n_hot]
        cur += n_hot
    dev_pages = np.concatenate(dev_pages, 0) if dev_pages else np.zeros((0, 3), np.int64)

    src = np.zeros(R, dtype=np.int64) if spec.shared_src else np.arange(R, dtype=np.int64) + 1

    # host blocks: every page completed initially (shared between requests when
    # they read one source), then one private block per page completed during the run
    done0 = ctx0 // PAGE
    done_final = ctx_final // PAGE
    hbt = np.full((R, max_pages), -1, dtype=np.int32)
    n_init = int(done0.max()) if spec.shared_src else int(done0.sum())
    n_run = int((done_final - done0).sum())
    n_host = n_init + n_run
    hperm = rng.permutation(rng.key(seed, 0x4057), max(1, n_host)).astype(np.int64)
    hp, hs = [], []
    if spec.shared_src:
        for r in range(R):
            hbt[r, :done0[r]] = hperm[:done0[r]]
        hp.append(np.stack([hperm[:n_init], np.arange(n_init)], 1))
        hs.append(np.zeros(n_init, dtype=np.int64))
    else:
        base = 0
        for r in range(R):
            ids = hperm[base:base + done0[r]]
            base += int(done0[r])
            hbt[r, :done0[r]] = ids
            hp.append(np.stack([ids, np.arange(done0[r])], 1))
            hs.append(np.full(done0[r], src[r]))
    host_pages = np.concatenate(hp, 0) if hp else np.zeros((0, 2), np.int64)
    host_src = np.concatenate(hs) if hs else np.zeros(0, np.int64)
    run_base = np.cumsum(np.concatenate([[n_init], (done_final - done0)]))

    def host_of(r, p):
        return int(hperm[run_base[r] + (p - done0[r])])

    classes = spec.classes.astype(np.int8)
    wl = Workload(name=spec.name, seed=seed, R=R, L=L, P=P, K=K, C=C, n_blocks=n_blocks,
                  n_host_blocks=max(1, n_host), max_pages=max_pages,
                  ctx0=ctx0.astype(np.int32), block_table=bt.copy(),
                  host_block_table=hbt.copy(), hot_blocks=hot, src=src,
                  dev_pages=dev_pages, host_pages=host_pages.astype(np.int64),
                  host_src=host_src, classes=classes, G=G)

    # steps
    ov_n, rc_n, un_n = _split_counts(K, spec.mix)
    prev = [[None] * NG for _ in range(R)]
    cur_bt = bt.copy()
    cur_hbt = hbt.copy()
    pend_hbt = []     # host-table entries that become valid after the previous step's offload
    for s in range(spec.steps):
        ctx = ctx_steps[s]
        # pages that left the tail are nulled before the step; they must have host copies
        bt_set = []
        for r in range(R):
            for p in range(int(fr0[r]) if s == 0 else int(fr_steps[s - 1][r]), int(fr_steps[s][r])):
                if cur_bt[r, p] != -1:
                    bt_set.append((r, p, -1))
        hbt_set = pend_hbt
        for (r, p, v) in hbt_set:
            cur_hbt[r, p] = v
        for (r, p, v) in bt_set:
            if cur_hbt[r, p] == -1:
                raise AssertionError("a page is nulled before its host copy exists")
            cur_bt[r, p] = v
        topk = np.full((R, NG, P, K), -1, dtype=np.int32)
        for r in range(R):
            c = int(ctx[r])
            for layer in range(NG):  # a layer group's list (one group per layer if G = 1)
                kk = rng.key(seed, 0x70C, s, r, layer)
                p0 = _mix(kk, prev[r][layer], c, K, ov_n, rc_n, spec.recent_window,
                          spec.first_recent_share)
                prev[r][layer] = p0
                topk[r, layer, 0] = p0
                for pos in range(1, P):
                    kp = rng.key(kk, 0x905, pos)
                    keep = _sample(rng.key(kp, 1), p0, spec.pos_keep)
                    fresh = K - spec.pos_keep
                    f_rc = int(math.floor(fresh * spec.first_recent_share))
                    rc = _distinct(rng.key(kp, 2), f_rc, max(0, c - spec.recent_window), c, keep)
                    un = _distinct(rng.key(kp, 3), fresh - f_rc, 0, c, np.concatenate([keep, rc]))
                    topk[r, layer, pos] = _shuffle(rng.key(kp, 4), np.concatenate([keep, rc, un]))
        # pages completed during this step get their proactive host copy afterwards
        prev_ctx = ctx0 if s == 0 else ctx_steps[s - 1]
        offload = []
        pend_hbt = []
        for r in range(R):
            lo_p = int(prev_ctx[r]) // PAGE if s > 0 else int(ctx0[r]) // PAGE
            for p in range(lo_p, int(ctx[r]) // PAGE):
                if cur_hbt[r, p] != -1:
                    continue
                hbv = host_of(r, p)
                if cur_bt[r, p] == -1:
                    raise AssertionError("completed page is neither resident nor on host")
                offload.append((int(cur_bt[r, p]), hbv))
                pend_hbt.append((r, p, hbv))
        wl.steps.append(Step(stamp=s + 1, ctx=ctx.astype(np.int32), topk=topk,
                             bt_set=np.array(bt_set, dtype=np.int64).reshape(-1, 3),
                             hbt_set=np.array(hbt_set, dtype=np.int64).reshape(-1, 3),
                             offload=np.array(offload, dtype=np.int32).reshape(-1, 2)))
    return wl


# ---------------------------------------------------------------------------
# the five workloads

def tiny(seed: int = 1000, steps: int = 4) -> Workload:
    """1 request, 1 layer, context 4096, top-K 256, hot buffer 512 rows; the
    last 1024 tokens are a resident tail; each step's top-K is half repeats of
    the previous step's set and half uniform; no tokens are appended."""
    return build(Spec(name="tiny", seed=seed, R=1, L=1, K=256, C=512, steps=steps,
                      ctx0=np.array([4096]), classes=np.array([1]), tail_frac=0.25,
                      append=0, append_first=False, mix=(0.5, 0.0, 0.5),
                      first_recent_share=0.0))


def mixed_decode(seed: int = 1001, steps: int = 16, R: int = 32) -> Workload:
    """32 requests x 1 layer at 74,160 tokens, 25 % resident tail, top-K 2048,
    hot buffer 4096; +1 token per step; 70 % overlap / 20 % last 4096 / 10 %
    uniform."""
    return build(Spec(name="mixed_decode", seed=seed, R=R, L=1, K=2048, C=4096,
                      steps=steps, ctx0=np.full(R, 74160), classes=np.ones(R, np.int8),
                      tail_frac=0.25))


def multi_layer(seed: int = 1002, turns: int = 13, R: int = 64, L: int = 16) -> Workload:
    """64 requests x 16 layers, contexts uniform in [74,160, 142,000], +753
    tokens per turn, one resolve per turn, 10 % resident tail that moves with
    the context; pages completed in a turn are copied to host after it.  All
    requests read one source sequence so that one host copy per page serves
    every request (keeps the host pool at ~1.6 GB instead of ~73 GB)."""
    ctx0 = rng.uniform_ints(rng.key(seed, 0xC7), 0, R, 74160, 142001)
    return build(Spec(name="multi_layer", seed=seed, R=R, L=L, K=2048, C=4096, steps=turns,
                      ctx0=ctx0, classes=np.ones(R, np.int8), tail_frac=0.10,
                      append=753, append_first=False, shared_src=True, move_tail=True))


def no_residency(seed: int = 1003, steps: int = 32, R: int = 8) -> Workload:
    """8 requests reusing one host-only 1,000,000-token prefix; one real page
    takes the decode tokens; empty hot buffer of 4096; top-K 2048; step 0 is
    uniform (all misses), later steps 80 % overlap + 20 % uniform."""
    return build(Spec(name="no_residency", seed=seed, R=R, L=1, K=2048, C=4096, steps=steps,
                      ctx0=np.full(R, 1_000_000), classes=np.full(R, 2, np.int8),
                      mix=(0.80, 0.0, 0.20), first_recent_share=0.0, shared_src=True))


def mixed_state(seed: int = 1004, steps: int = 16, R: int = 128) -> Workload:
    """128 requests, 40 % full / 40 % mixed (25 % tail) / 20 % no residency,
    contexts log-uniform in [8192, 1,000,000], top-K 2048, hot buffer 4096,
    4 query positions per step resolved as one plan; +1 token per step."""
    u = (rng.draws(rng.key(seed, 0xC7), 0, R) >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    ctx0 = np.floor(np.exp(np.log(8192.0) + u * (np.log(1e6) - np.log(8192.0)))).astype(np.int64)
    n_full, n_mixed = int(math.floor(0.4 * R)), int(math.floor(0.4 * R))
    cls = np.array([0] * n_full + [1] * n_mixed + [2] * (R - n_full - n_mixed), dtype=np.int8)
    cls = cls[rng.permutation(rng.key(seed, 0xC1A5), R)]
    return build(Spec(name="mixed_state", seed=seed, R=R, L=1, K=2048, C=4096, steps=steps,
                      ctx0=ctx0, classes=cls, tail_frac=0.25, P=4, shared_src=True))


def mtp_state(seed: int = 1004, steps: int = 16, R: int = 128) -> Workload:
    """mixed_state with the hot buffer sized for speculative decoding (the
    note on multi-token prediction in the section that estimates the effect
    for a configuration: every verified token must fit at once, (speculative
    tokens + 2) x top-K rows): 3 speculative tokens, a 4-position plan,
    5 x 2048 = 10,240 slots per request; the same contexts, classes and lists
    as mixed_state."""
    u = (rng.draws(rng.key(seed, 0xC7), 0, R) >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    ctx0 = np.floor(np.exp(np.log(8192.0) + u * (np.log(1e6) - np.log(8192.0)))).astype(np.int64)
    n_full, n_mixed = int(math.floor(0.4 * R)), int(math.floor(0.4 * R))
    cls = np.array([0] * n_full + [1] * n_mixed + [2] * (R - n_full - n_mixed), dtype=np.int8)
    cls = cls[rng.permutation(rng.key(seed, 0xC1A5), R)]
    return build(Spec(name="mtp_state", seed=seed, R=R, L=1, K=2048, C=5 * 2048, steps=steps,
                      ctx0=ctx0, classes=cls, tail_frac=0.25, P=4, shared_src=True))


def grouped_decode(seed: int = 1005, steps: int = 16, R: int = 32, L: int = 4,
                   G: int = 4) -> Workload:
    """mixed_decode with IndexShare ("Use sparsity when needed": one indexer
    layer per 4 sparse-MLA layers): 32 requests x 4 layers forming one group
    that shares each step's top-K list and one hot buffer; 74,160 tokens, 25 %
    resident tail, top-K 2048, hot buffer 4096, +1 token per step."""
    return build(Spec(name="grouped_decode", seed=seed, R=R, L=L, K=2048, C=4096, steps=steps,
                      ctx0=np.full(R, 74160), classes=np.ones(R, np.int8), tail_frac=0.25,
                      group=G))


def build_dynamic(spec: Spec, residency, n_blocks: int, host_base: int) -> Workload:
    """A workload whose residency is decided step by step by ``residency``
    instead of being scripted: contexts and top-K lists are drawn as in
    ``build`` (they do not depend on residency); ``residency`` is any object
    with ``admit(r, ctx, host_block_of_page)`` and ``step(stamp, reqs, ctx,
    topk)`` returning edits with ``bt_set``, ``hbt_set``, ``hot_set``,
    ``reset`` and ``offload`` (the residency policy's, in the tests);
    ``admit`` also takes whether the prefix starts resident (class 0).  Each
    request starts with the host copies of its complete pages (a reused
    prefix), in host blocks ``host_base`` and up (the decider's own host
    blocks lie below); the decider chooses what stays resident."""
    R, L, P, K, C = spec.R, spec.L, spec.P, spec.K, spec.C
    if P != 1 or C % PAGE:
        raise ValueError("one query position per step and whole-page hot buffers")
    G = spec.group
    NG = L // G
    seed = spec.seed
    ctx0 = spec.ctx0.astype(np.int64)
    ctx_steps = [ctx0 + (s + 1) * spec.append for s in range(spec.steps)]
    ctx_final = ctx_steps[-1] if spec.steps else ctx0
    max_pages = int(((ctx_final + PAGE - 1) // PAGE).max())
    src = np.arange(R, dtype=np.int64) + 1
    # the reused prefix: host copies of the complete pages, private per request
    done0 = ctx0 // PAGE
    host_of_page = []
    host_pages, host_src = [], []
    base = host_base
    for r in range(R):
        ids = np.arange(base, base + int(done0[r]), dtype=np.int64)
        base += int(done0[r])
        host_of_page.append(ids.astype(np.int32))
        host_pages.append(np.stack([ids, np.arange(done0[r])], 1))
        host_src.append(np.full(done0[r], src[r]))
    n_host_blocks = base
    bt = np.full((R, max_pages), -1, np.int32)
    hbt = np.full((R, max_pages), -1, np.int32)
    hot = np.full((R, C // PAGE), -1, np.int32)
    dev_pages = []
    for r in range(R):
        # class 0: the prefix stays resident (with its host copy); else host-only
        e = residency.admit(r, int(ctx0[r]), host_of_page[r], bool(spec.classes[r] == 0))
        for rr, p, v in e.hbt_set:
            hbt[rr, p] = v
        for rr, p, v in e.bt_set:
            bt[rr, p] = v
            if v >= 0:
                dev_pages.append((rr, p, v))
        for rr, j, v in e.hot_set:
            hot[rr, j] = v
    wl = Workload(name=spec.name, seed=seed, R=R, L=L, P=P, K=K, C=C, n_blocks=n_blocks,
                  n_host_blocks=n_host_blocks, max_pages=max_pages, ctx0=ctx0.astype(np.int32),
                  block_table=bt, host_block_table=hbt, hot_blocks=hot, src=src,
                  dev_pages=np.array(dev_pages, np.int64).reshape(-1, 3),
                  host_pages=np.concatenate(host_pages, 0).astype(np.int64),
                  host_src=np.concatenate(host_src).astype(np.int64),
                  classes=spec.classes.astype(np.int8), G=G)
    ov_n, rc_n, _ = _split_counts(K, spec.mix)
    prev = [[None] * NG for _ in range(R)]
    last = None
    for s in range(spec.steps):
        ctx = ctx_steps[s]
        e = residency.step(s + 1, np.arange(R), ctx.astype(np.int32), last)
        topk = np.full((R, NG, P, K), -1, dtype=np.int32)
        for r in range(R):
            c = int(ctx[r])
            for g in range(NG):
                kk = rng.key(seed, 0x70C, s, r, g)
                p0 = _mix(kk, prev[r][g], c, K, ov_n, rc_n, spec.recent_window,
                          spec.first_recent_share)
                prev[r][g] = p0
                topk[r, g, 0] = p0
        # the decider warms pages by every list of the step (all groups)
        last = topk.reshape(R, -1)
        new_pages = np.array([(r, p, v) for r, p, v in e.bt_set if v >= 0],
                             np.int64).reshape(-1, 3)
        wl.steps.append(Step(stamp=s + 1, ctx=ctx.astype(np.int32), topk=topk,
                             bt_set=np.asarray(e.bt_set, np.int64).reshape(-1, 3),
                             hbt_set=np.asarray(e.hbt_set, np.int64).reshape(-1, 3),
                             offload=np.asarray(e.offload, np.int32).reshape(-1, 2),
                             hot_set=np.asarray(e.hot_set, np.int64).reshape(-1, 3),
                             reset=np.asarray(e.reset, np.int64).reshape(-1),
                             new_pages=new_pages))
    return wl


def ungrouped(wl: Workload) -> Workload:
    """The same workload with one group per layer: each layer gets its group's
    top-K list (and, when run, a hot-buffer state of its own) -- the per-layer
    alternative a grouped resolve replaces."""
    import copy
    if wl.G == 1:
        return wl
    out = copy.copy(wl)
    out.name = wl.name + "_per_layer"
    out.G = 1
    out.steps = [Step(stamp=s.stamp, ctx=s.ctx, topk=np.repeat(s.topk, wl.G, axis=1),
                      bt_set=s.bt_set, hbt_set=s.hbt_set, offload=s.offload) for s in wl.steps]
    return out


CONFIGS = {
    "tiny": tiny,
    "mixed_decode": mixed_decode,
    "multi_layer": multi_layer,
    "no_residency": no_residency,
    "mixed_state": mixed_state,
    "grouped_decode": grouped_decode,
    "mtp_state": mtp_state,
}
