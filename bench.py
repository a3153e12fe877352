#!/usr/bin/env python3
"""Benchmark of the Hybrid HiSparse hot path on one MI355X.

A step is one pass of the whole hot path over one decode batch of the
mixed-residency workload (32 requests x 1 layer at a 74,160-token context,
25 % resident tail, top-K 2048, 4096 hot rows per request, +1 token per
step): the fused resolver (classify, hit refresh, LRU victims, one-row host
copies of the misses, state commit), the single-stride gather of all
65,536 rows, and -- in the steps where a page completes -- the batched
prefix-page offload.  Inputs (top-K lists, tables, pools) are resident in
device / pinned host memory before the timed region.

Prints one JSON line: resolved top-K rows/s for the whole job, plus the
roofline of the dominant kernel (per-launch duration from HIP events on the
kernel's own stream, algorithmic bytes per launch), the achieved HBM and host-link
bandwidths, a hit-replay measurement of the HBM-bound path, and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "resolved top-K rows/s + achieved HBM & host-link GB/s vs peak, 32 req x K=2048"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA
HOST_LINK_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction
ROW = 656
PAGE = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="mixed_decode",
                    choices=["mixed_decode", "no_residency", "mixed_state", "mtp_state",
                             "multi_layer", "grouped_decode", "grouped_decode_per_layer"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hit-replays", type=int, default=50)
    ap.add_argument("--serial", action="store_true",
                    help="time the serial stages (decide, then move with the host copies) "
                         "instead of the overlapped hs_plan_replay")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying a captured graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain 256 MiB device copy (counter calibration runs)")
    ap.add_argument("--consumer", action=argparse.BooleanOptionalAction, default=True,
                    help="also time a decode step consumed by sparse MLA attention, gathered "
                         "and in place")
    ap.add_argument("--miss-path", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the all-miss first step of the no-residency workload "
                         "(every row over the host link)")
    ap.add_argument("--ceilings", action=argparse.BooleanOptionalAction, default=True,
                    help="also probe the HBM copy and host-link DMA ceilings in the same job")
    ap.add_argument("--cold-steps", type=int, default=16,
                    help="steps after the event-timed ones, each behind an untimed 1 GiB scrub "
                         "(cold caches: the 256 MB MALL and the L2s hold nothing of the step)")
    ap.add_argument("--event-steps", type=int, default=64,
                    help="steps launched one by one with HIP events around every kernel "
                         "(per-kernel durations), after the timed steps")
    return ap.parse_args()


def build_workload(name: str, n_steps: int):
    import hs_gen
    if name == "mixed_decode":
        return hs_gen.mixed_decode(steps=n_steps)
    if name == "no_residency":
        return hs_gen.no_residency(steps=n_steps)
    if name == "mixed_state":
        return hs_gen.mixed_state(steps=n_steps)
    if name == "mtp_state":
        return hs_gen.mtp_state(steps=n_steps)
    if name == "grouped_decode":
        return hs_gen.grouped_decode(steps=n_steps)
    if name == "grouped_decode_per_layer":
        return hs_gen.ungrouped(hs_gen.grouped_decode(steps=n_steps))
    return hs_gen.multi_layer(turns=n_steps)


def kernel_source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the kernel sources, in name
    order, with comments and blank space taken out (so a comment edit leaves
    measured figures valid; any change to the code does not)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "serving_memory_tier_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when it was taken on another workload or on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = fields.get(f"{kernel}_traffic_bytes_per_launch")
    return int(v) if v else None


def decide_hbm_bytes(wl, stats_sum, n_launches):
    """Algorithmic HBM bytes of the decision kernel per launch.

    Per request-layer (per layer group when layers share lists): the slot
    tokens and stamps are read once (8 B/slot).  Per entry: the index (4 B),
    its block-table entry (4 B), its row (4 B).  Per hit: the refreshed stamp
    (4 B).  Per miss: the host-table entry (4 B) and the slot's new token and
    stamp (8 B).
    """
    R, NG, N = wl.R, wl.NG, wl.P * wl.K
    hits, misses = stats_sum[1], stats_sum[2]
    return R * NG * wl.C * 8 + R * NG * N * 12 + (hits * 4 + misses * 12) / n_launches


def fetch_bytes(wl, stats_sum, n_launches):
    """(host-link bytes, HBM bytes) of the early fill's rows per launch: every
    distinct miss (assigned or not) reads its 656-B row over the host link;
    every resident or hit entry reads its 656-B row from the pool; every entry
    writes its 656-B output row.  The fill's reads of the entries, tables and
    slot tokens are the resolver's reads again (L2 hits in the fused launch)
    and are counted once, in decide_hbm_bytes.  With layer groups every miss
    and every row is moved once per layer of the group."""
    R, L, N = wl.R, wl.L, wl.P * wl.K
    entries = R * L * N
    m = (stats_sum[2] + stats_sum[3]) / n_launches * wl.G
    return m * ROW, (entries - m) * ROW + entries * ROW


def commit_bytes(wl, stats_sum, n_launches):
    """HBM bytes of the commit per launch: every entry's code (4 B); per
    assigned miss its row read from the output and written into the slot, the
    slot's token and the final row id (the rows once per layer of a group)."""
    R, NG, N = wl.R, wl.NG, wl.P * wl.K
    a = stats_sum[2] / n_launches
    return R * NG * N * 4 + a * (2 * ROW * wl.G + 8)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(request-layers are independent, so a data-parallel run would be N copies "
              "of this measurement).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import serving_memory_tier_amd as hs
    from serving_memory_tier_amd.hipgraph import HipRuntime
    from serving_memory_tier_amd.runner import DeviceRun

    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    torch.cuda.set_device(0)

    W, K = args.warmup, args.steps
    KE = min(K, args.event_steps)  # eager steps timed with events, after the graph
    NC = max(0, args.cold_steps)   # then steps behind a cache scrub, timed the same way
    t_gen = time.time()
    wl = build_workload(args.workload, W + K + KE + NC)
    print(f"[bench] workload {wl.name}: R={wl.R} L={wl.L} P={wl.P} K={wl.K} C={wl.C} "
          f"steps={len(wl.steps)} generated in {time.time() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    dev = DeviceRun(wl)
    dev.upload_steps()
    n_steps = len(wl.steps)
    N = wl.P * wl.K
    entries = wl.R * wl.L * N
    dev.stage_steps()
    stats_all = torch.zeros((n_steps, wl.R, wl.NG, 8), dtype=torch.int32, device="cuda")
    hev = HipRuntime()

    def step(i, sp):
        dev.launch_step(i, hev, sp, stats=stats_all[i], serial=args.serial)

    sp0 = torch.cuda.current_stream().cuda_stream
    for i in range(W):
        step(i, sp0)
    torch.cuda.synchronize()
    launch = "eager"
    graph = False
    cap = torch.cuda.Stream()
    if not args.eager:
        # the K timed steps, captured once and replayed as one graph: the
        # decode path waits on nothing from the host, so it captures as is
        try:
            hev.begin_capture(cap.cuda_stream)
            try:
                for j in range(K):
                    step(W + j, cap.cuda_stream)
            finally:
                hev.end_capture(cap.cuda_stream)
            graph = True
            launch = "hip_graph"
        except Exception as exc:  # fall back to eager launches
            print(f"[bench] graph capture failed ({exc}); timing eager launches",
                  file=sys.stderr, flush=True)
            graph = False
    if graph:
        hev.upload(cap.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph:
        hev.launch(cap.cuda_stream)
    else:
        for j in range(K):
            step(W + j, sp0)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    hev.destroy_graph()

    # per-kernel durations: the next KE steps launched as hs_plan_replay's
    # stages on the launch stream (the fused resolve-and-fill launch, the
    # commit, the offload), HIP events on that stream around every kernel.
    # The events before the offload release to device scope only (a
    # system-scope release at each record adds about a microsecond to the
    # kernel it closes); the one after it, whose kernel writes host memory,
    # keeps the system scope.
    def step_events():
        return [hev.new_event(system_fence=False) for _ in range(3)] + [hev.new_event()]

    events = [step_events() for _ in range(KE)]
    busy = QueueFiller()
    for j in range(KE):
        busy.fill()
        dev.launch_step_timed(W + K + j, hev, sp0, events[j], stats=stats_all[W + K + j])
    torch.cuda.synchronize()

    def mean_us(a, b, ev=events, n=KE):
        # the median: a launch the host enqueued late (after the device spin
        # ahead of it ran out) would add its host delay to the mean
        return 1e3 * float(np.median([hev.elapsed_ms(ev[j][a], ev[j][b]) for j in range(n)]))

    fused_us, commit_us = mean_us(0, 1), mean_us(1, 2)
    off = [(j, hev.elapsed_ms(events[j][2], events[j][3])) for j in range(KE)
           if wl.steps[W + K + j].offload.shape[0]]
    st = stats_all[W + K:W + K + KE].sum(dim=(0, 1, 2)).cpu().numpy().astype(np.int64)
    st_all = stats_all[W:W + K].sum(dim=(0, 1, 2)).cpu().numpy().astype(np.int64)
    value = entries * K / wall

    f_host, f_hbm = fetch_bytes(wl, st, KE)
    fused_hbm = decide_hbm_bytes(wl, st, KE) + f_hbm
    com_bytes = commit_bytes(wl, st, KE)
    kernels = {
        "resolve_fill": {"us": round(fused_us, 2), "host_link_bytes": int(f_host),
                         "host_link_gbps": round(f_host / fused_us / 1e3, 2),
                         "hbm_bytes": int(fused_hbm),
                         "hbm_gbps": round(fused_hbm / fused_us / 1e3, 1)},
        "commit": {"us": round(commit_us, 2), "hbm_bytes": int(com_bytes),
                   "hbm_gbps": round(com_bytes / max(commit_us, 1e-3) / 1e3, 1)},
    }
    if wl.G > 1:
        # one event pair spans the whole hs_resolve_grouped call
        kernels["resolve_fill"]["note"] = ("layer groups of %d: the whole hs_resolve_grouped call "
                                           "(fused launch, commit, offload)" % wl.G)
        kernels.pop("commit")
        kernels.pop("offload", None)
    if off:
        page_layers = [wl.steps[W + K + j].offload.shape[0] * wl.L for j, _ in off]
        off_us = 1e3 * float(np.median([ms for _, ms in off]))
        off_bytes = float(np.mean(page_layers)) * PAGE * ROW
        kernels["offload"] = {"us": round(off_us, 2), "launches": len(off),
                              "host_link_bytes": int(off_bytes),
                              "host_link_gbps": round(off_bytes / off_us / 1e3, 2)}

    # cold steps: each behind an untimed write of 1 GiB, so that no cache holds
    # the step's lists, tables, state or rows
    cold = None
    if NC:
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cev = [step_events() for _ in range(NC)]
        cst = torch.zeros((NC, wl.R, wl.NG, 8), dtype=torch.int32, device="cuda")
        for j in range(NC):
            scrub.fill_(j & 0xFF)
            busy.fill()
            dev.launch_step_timed(W + K + KE + j, hev, sp0, cev[j], stats=cst[j])
        torch.cuda.synchronize()
        del scrub
        sc = cst.sum(dim=(0, 1, 2)).cpu().numpy().astype(np.int64)
        c_fused, c_commit = mean_us(0, 1, cev, NC), mean_us(1, 2, cev, NC)
        c_host = fetch_bytes(wl, sc, NC)[0]
        cold = {"steps": NC, "resolve_fill_us": round(c_fused, 2),
                "commit_us": round(c_commit, 2), "step_us": round(c_fused + c_commit, 2),
                "host_link_gbps": round(c_host / c_fused / 1e3, 2),
                "rows_per_s": round(entries / ((c_fused + c_commit) * 1e-6)),
                "note": "each step behind an untimed 1 GiB scrub; warm figures are 'kernels'"}

    # the hit-replay path: the last step's lists again with the same stamp --
    # every non-resident token hits, no host traffic, HBM-bound
    last = W + K + KE + NC - 1
    NR = args.hit_replays
    rep = [step_events() for _ in range(NR)]
    rep_stats = torch.zeros((wl.R, wl.NG, 8), dtype=torch.int32, device="cuda")
    for j in range(NR):
        busy.fill()
        dev.launch_step_timed(last, hev, sp0, rep[j], stats=rep_stats, offload=False)
    torch.cuda.synchronize()
    rs = rep_stats.sum(dim=(0, 1)).cpu().numpy()
    r_fused, r_commit = mean_us(0, 1, rep, NR), mean_us(1, 2, rep, NR)
    r_step = mean_us(0, 2, rep, NR)
    r_fused_bytes = decide_hbm_bytes(wl, rs, 1) + fetch_bytes(wl, rs, 1)[1]
    rep_bytes = r_fused_bytes + commit_bytes(wl, rs, 1)
    hit_replay = {"resolve_fill_us": round(r_fused, 2), "commit_us": round(r_commit, 2),
                  "step_us": round(r_step, 2), "misses": int(rs[2]),
                  "rows_per_s": round(entries / (r_step * 1e-6)),
                  "hbm_gbps": round(rep_bytes / r_step / 1e3, 1),
                  "hbm_frac": round(rep_bytes / r_step / 1e3 / HBM_PEAK_GBPS, 4),
                  "resolve_fill_hbm_gbps": round(r_fused_bytes / r_fused / 1e3, 1)}
    if graph and NR:
        # the same replays captured once and replayed as one graph, timed like
        # the decode steps (no event pairs between the launches): a hit
        # replay leaves the state as it found it, so replaying it is exact
        hev.begin_capture(cap.cuda_stream)
        try:
            for j in range(NR):
                dev.launch_step(last, hev, cap.cuda_stream, stats=rep_stats, offload=False)
        finally:
            hev.end_capture(cap.cuda_stream)
        torch.cuda.synchronize()
        # one untimed launch first: a graph's first launch also uploads it
        hev.launch(cap.cuda_stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        hev.launch(cap.cuda_stream)
        torch.cuda.synchronize()
        g_step = (time.perf_counter() - t2) / NR * 1e6
        hev.destroy_graph()
        hit_replay["graph_step_us"] = round(g_step, 2)
        hit_replay["graph_rows_per_s"] = round(entries / (g_step * 1e-6))
        hit_replay["graph_hbm_gbps"] = round(rep_bytes / g_step / 1e3, 1)
        hit_replay["graph_hbm_frac"] = round(rep_bytes / g_step / 1e3 / HBM_PEAK_GBPS, 4)
    regather = None
    if graph and NR and wl.G == 1:
        # the plan's rows gathered again for a further forward pass
        # (hs_gather over the last step's row ids), NR launches captured once
        # and timed like the hit replays
        valid = int(((dev.rows >= 0) & (dev.rows < wl.pool_rows)).sum().item())
        g_bytes = entries * 4 + entries * ROW + valid * ROW
        hev.begin_capture(cap.cuda_stream)
        try:
            for j in range(NR):
                dev.gather(cap.cuda_stream)
        finally:
            hev.end_capture(cap.cuda_stream)
        torch.cuda.synchronize()
        hev.launch(cap.cuda_stream)          # untimed first launch
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        hev.launch(cap.cuda_stream)
        torch.cuda.synchronize()
        g_us = (time.perf_counter() - t2) / NR * 1e6
        hev.destroy_graph()
        regather = {"graph_us": round(g_us, 2), "hbm_bytes": g_bytes,
                    "hbm_gbps": round(g_bytes / g_us / 1e3, 1),
                    "hbm_frac": round(g_bytes / g_us / 1e3 / HBM_PEAK_GBPS, 4),
                    "note": "hs_gather of the last step's row ids (the multi-forward replay of a "
                            "resolved plan), graph replay"}

    # page coldness for the residency policy: hs_page_touch over the last
    # step's lists, HIP events around each launch
    page_touch = touch_cost(wl, dev, hev, sp0, last, n=20, busy=busy)
    consumer = None
    if args.consumer and wl.G == 1 and wl.L == 1:
        consumer = consumer_cost(wl, hev, sp0, busy, n_steps=min(16, len(wl.steps)))
    miss_path = miss_path_cost(hev, sp0, busy) if args.miss_path else None
    ceilings = probe_ceilings(hev, sp0, busy) if args.ceilings else None
    busy.close()
    kernels["page_touch"] = page_touch
    policy = policy_cost(wl, dev)

    # the dominant kernel of a step -- the fused resolve-and-fill launch -- and
    # the resource that bounds it: the host link while it carries misses (its
    # HBM bytes would take a fraction of the time at HBM speed), HBM otherwise
    host_t = f_host / (HOST_LINK_PEAK_GBPS * 1e3)
    hbm_t = fused_hbm / (HBM_PEAK_GBPS * 1e3)
    if host_t >= hbm_t:
        ach = f_host / fused_us / 1e3
        roofline = {"kernel": "resolve_fill", "bound": "host_link", "achieved": round(ach, 2),
                    "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / HOST_LINK_PEAK_GBPS, 4), "traffic": None}
    else:
        ach = fused_hbm / fused_us / 1e3
        roofline = {"kernel": "resolve_fill", "bound": "hbm", "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "traffic": None}
    roofline["traffic"] = measured_traffic(roofline["kernel"], wl.name)
    if ceilings:
        # the same against what this chip's copies reach in this job
        ceil = (ceilings["host_to_device_dma_gbps"] if roofline["bound"] == "host_link"
                else ceilings["hbm_copy_gbps"])
        roofline["probed_ceiling"] = ceil
        roofline["frac_of_probed"] = round(roofline["achieved"] / ceil, 4)
        if miss_path:
            miss_path["host_link_frac_of_probed"] = round(
                miss_path["host_link_gbps"] / ceilings["host_to_device_dma_gbps"], 4)
        hit_replay["hbm_frac_of_probed"] = round(hit_replay["hbm_gbps"] / ceilings["hbm_copy_gbps"], 4)
        if "graph_hbm_gbps" in hit_replay:
            hit_replay["graph_hbm_frac_of_probed"] = round(
                hit_replay["graph_hbm_gbps"] / ceilings["hbm_copy_gbps"], 4)
    # whole steps of the timed region: algorithmic bytes per step / step time
    step_hbm_k = (decide_hbm_bytes(wl, st_all, K) + fetch_bytes(wl, st_all, K)[1] +
                  commit_bytes(wl, st_all, K))
    host_k = fetch_bytes(wl, st_all, K)[0]
    line = {
        "metric": METRIC, "value": round(value), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(1e3 * wall / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.R, "layers": wl.L, "positions": wl.P,
                   "top_k": wl.K, "hot_capacity": wl.C, "context": int(wl.ctx0.max()),
                   "row_bytes": ROW, "page_size": PAGE, "layer_group": wl.G, "launch": launch},
        "hbm": {"achieved": round(step_hbm_k / (wall / K) / 1e9, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(step_hbm_k / (wall / K) / 1e9 / HBM_PEAK_GBPS, 4)},
        "host_link": {"achieved": round(host_k / (wall / K) / 1e9, 2),
                      "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(host_k / (wall / K) / 1e9 / HOST_LINK_PEAK_GBPS, 4)},
        "per_step": {"hits": round(st_all[1] / K, 1), "misses": round(st_all[2] / K, 1),
                     "resident": round(st_all[0] / K, 1)},
        "kernels": kernels,
        "kernel_timing": f"HIP events on the launch stream around every kernel, median over "
                         f"{KE} steps launched as hs_plan_replay's stages after the timed ones, "
                         f"each queued behind a 0.3 ms device spin so no event waits on the host",
        "cold": cold,
        "hit_replay": hit_replay,
        "plan_regather": regather,
        "policy": policy,
        "consumer": consumer,
        "miss_path": miss_path,
        "ceilings": ceilings,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    hev.close()
    dev.close()
    if args.calibrate_copy:
        # a plain copy kernel of known size: 256 MiB read + 256 MiB written
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


class QueueFiller:
    """A ~0.3 ms spin on the device (no memory traffic, so caches stay as the
    previous kernels left them) enqueued ahead of a timed launch sequence:
    the host has queued the whole sequence before the GPU reaches its first
    event, so the events time the kernels, not the host's launch calls."""

    def __init__(self, target_us: float = 300.0):
        import torch
        probe = 1 << 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(probe)          # first call loads the kernel
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(probe)
        b.record()
        torch.cuda.synchronize()
        us_per_cycle = a.elapsed_time(b) * 1e3 / probe
        self.cycles = int(max(1 << 14, min(1 << 30, target_us / max(us_per_cycle, 1e-9))))

    def fill(self) -> None:
        import torch
        torch.cuda._sleep(self.cycles)

    def close(self) -> None:
        pass


def consumer_cost(wl, hev, stream: int, busy, n_steps: int = 16, heads: int = 128):
    """A decode step consumed by sparse MLA attention (128 heads, 576-wide
    queries) two ways, over the workload's first n_steps steps, each on a
    fresh copy of the batch: the resolver with its gathered output and the
    attention over the gathered rows, or the resolver in place
    (hs_resolve_in_place: only the misses staged) and the attention reading
    the pool by row id.  HIP events around the resolve and the attention of
    every step; each step queued behind a device spin."""
    import math

    import numpy as np
    import torch

    import serving_memory_tier_amd as hs
    from serving_memory_tier_amd.runner import DeviceRun
    # one query token per (request, position), each attending to its own K rows
    T, K = wl.R * wl.P, wl.K
    q = (torch.randn((T, heads, 576), device="cuda") * 0.5).to(torch.bfloat16).view(torch.int16)
    out = torch.empty((T, heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, heads), dtype=torch.float32, device="cuda")
    wsb = hs.hs_sparse_mla_workspace_bytes(T, heads, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    iota = torch.arange(T * K, dtype=torch.int32, device="cuda").view(T, K)
    scale = 1.0 / math.sqrt(576)
    res = {}
    for mode in ("gathered", "in_place"):
        dev = DeviceRun(wl)
        dev.upload_steps()
        # the kernel reads T x K row ids, and in the gathered mode T x K rows
        assert dev.rows.numel() == T * K and dev.out.shape[:-1].numel() == T * K, \
            "consumer shapes must match the batch's row ids and gathered rows"
        assert dev.out.shape[-1] == ROW
        lay_kv = hs.layout_of(1, ROW, 1, 64, wl.pool_rows if mode == "in_place" else T * K, 0)
        # the middle event closes a call whose offload writes host memory
        ev = [(hev.new_event(system_fence=False), hev.new_event(), hev.new_event(system_fence=False))
              for _ in range(n_steps)]
        for i in range(n_steps):
            s = wl.steps[i]
            dev.pre(i)
            torch.cuda.synchronize()
            busy.fill()
            n_off = s.offload.shape[0]
            hev.record(ev[i][0], stream)
            if mode == "in_place":
                hs.hs_resolve_in_place(dev.layout, dev.batch, dev.topk[i], wl.P, wl.K, s.stamp,
                                       dev.rows, dev.out, dev.stats,
                                       dev.pairs[i] if n_off else None, n_off, stream)
                hev.record(ev[i][1], stream)
                hs.hs_sparse_mla_decode(lay_kv, dev.pool, dev.rows, T, K, q, heads, scale, out,
                                        lse, ws, wsb, stream)
            else:
                hs.hs_plan_replay(dev.layout, dev.batch, dev.topk[i], wl.P, wl.K, s.stamp,
                                  dev.rows, dev.out, dev.stats, dev.pairs[i] if n_off else None,
                                  n_off, stream)
                hev.record(ev[i][1], stream)
                hs.hs_sparse_mla_decode(lay_kv, dev.out, iota, T, K, q, heads, scale, out, lse,
                                        ws, wsb, stream)
            hev.record(ev[i][2], stream)
        torch.cuda.synchronize()
        r_us = [1e3 * hev.elapsed_ms(a, b) for a, b, _ in ev]
        a_us = [1e3 * hev.elapsed_ms(b, c) for _, b, c in ev]
        res[mode] = {"resolve_us": round(float(np.median(r_us)), 2),
                     "attention_us": round(float(np.median(a_us)), 2),
                     "step_us": round(float(np.median(r_us) + np.median(a_us)), 2)}
        dev.close()
    flops = 2.0 * T * heads * K * (576 + 512)
    for mode in res:
        a = res[mode]["attention_us"]
        res[mode]["attention_tflops"] = round(flops / a / 1e6, 1)
        res[mode]["rows_per_s"] = round(T * K / (res[mode]["step_us"] * 1e-6))
    best = res["in_place"]["attention_tflops"]
    res["attention_roofline"] = {"kernel": "attend", "bound": "mfma", "achieved": best,
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(best / BF16_PEAK_TFLOPS, 4),
                                 "flops_per_launch": int(flops)}
    res["heads"] = heads
    res["note"] = ("decode step = resolve + sparse MLA attention; 'gathered' copies every "
                   "selected row into a gathered buffer first, 'in_place' reads the pool by row id")
    return res


def miss_path_cost(hev, stream: int, busy, reps: int = 8):
    """The miss path alone: the first step of the no-residency workload (8
    requests sharing a host-only 1,000,000-token prefix, top-K 2048, an empty
    4096-row hot buffer), where every one of the 16,384 entries is a distinct
    miss and every row crosses the host link.  Steps 0..reps-1 of the workload
    are each resolved from an empty hot buffer (state cleared off the clock),
    so every call is all misses; HIP events around the fused resolve-and-fill
    launch and the commit, each call queued behind a device spin."""
    import numpy as np
    import torch

    import hs_gen
    from serving_memory_tier_amd.runner import DeviceRun
    wl = hs_gen.no_residency(steps=reps)
    dev = DeviceRun(wl)
    dev.upload_steps()
    dev.stage_steps()
    ev = [[hev.new_event(system_fence=False) for _ in range(4)] for _ in range(reps)]
    stats = torch.zeros((reps, wl.R, wl.NG, 8), dtype=torch.int32, device="cuda")
    for j in range(reps):
        dev.tok.fill_(-1)
        dev.stp.zero_()
        busy.fill()
        dev.launch_step_timed(j, hev, stream, ev[j], stats=stats[j], offload=False)
    torch.cuda.synchronize()
    st = stats.sum(dim=(1, 2)).cpu().numpy().astype(np.int64)
    fused = np.array([1e3 * hev.elapsed_ms(e[0], e[1]) for e in ev])
    commit = np.array([1e3 * hev.elapsed_ms(e[1], e[2]) for e in ev])
    host_bytes = float(np.mean((st[:, 2] + st[:, 3]) * ROW))
    dev.close()
    f_us, c_us = float(np.median(fused)), float(np.median(commit))
    gbps = host_bytes / f_us / 1e3
    return {"workload": "no_residency first step (8 x 2048, empty 4096-row hot buffer)",
            "calls": reps, "misses": int(np.mean(st[:, 2])),
            "host_link_bytes": int(host_bytes), "resolve_fill_us": round(f_us, 2),
            "resolve_fill_us_first_call": round(float(fused[0]), 2),
            "commit_us": round(c_us, 2), "step_us": round(f_us + c_us, 2),
            "host_link_gbps": round(gbps, 2), "host_link_frac": round(gbps / HOST_LINK_PEAK_GBPS, 4),
            "step_host_link_gbps": round(host_bytes / (f_us + c_us) / 1e3, 2)}


def probe_ceilings(hev, stream: int, busy):
    """The chip's practical ceilings in the same job: a 1 GiB device-to-device
    copy (HBM read + write), and 256 MiB DMA copies from pinned host memory to
    the device and back (the host link, one direction each).  HIP events
    around each copy on the launch stream; best of three."""
    import torch

    def best(fn, nbytes, reps=3):
        t = []
        for _ in range(reps):
            a, b = hev.new_event(), hev.new_event()   # copies to and from host memory
            busy.fill()
            hev.record(a, stream)
            fn()
            hev.record(b, stream)
            torch.cuda.synchronize()
            t.append(hev.elapsed_ms(a, b))
        return nbytes / (min(t) * 1e-3) / 1e9

    # the copies go to torch's current stream, which must be the timed one
    assert torch.cuda.current_stream().cuda_stream == stream
    d0 = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    d1 = torch.empty_like(d0)
    d0.fill_(1)
    torch_copy = best(lambda: d1.copy_(d0), 2 << 30)
    # a plain streaming-copy kernel (libhs_probe.so), its best launch shape
    probe = _probe_lib()
    kern, kern_shape = 0.0, None
    for variant, grid in ((1, 256), (0, 256), (2, 256), (3, 4096), (1, 512)):
        rc = []
        r = best(lambda: rc.append(probe.hs_probe_copy(d0.data_ptr(), d1.data_ptr(), 1 << 30,
                                                       grid, variant, stream)), 2 << 30)
        assert all(x == 0 for x in rc), "copy probe launch failed"
        if r > kern:
            kern, kern_shape = r, f"variant {variant}, {grid} workgroups of 256"
    assert torch.equal(d0[:1 << 20], d1[:1 << 20])
    hbm = max(torch_copy, kern)
    del d0, d1
    h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    h2d = best(lambda: d.copy_(h, non_blocking=True), 256 << 20)
    d2h = best(lambda: h.copy_(d, non_blocking=True), 256 << 20)
    torch.cuda.synchronize()
    del h, d
    return {"hbm_copy_gbps": round(hbm, 1), "hbm_copy_kernel_gbps": round(kern, 1),
            "hbm_copy_kernel_shape": kern_shape, "torch_copy_gbps": round(torch_copy, 1),
            "host_to_device_dma_gbps": round(h2d, 2),
            "device_to_host_dma_gbps": round(d2h, 2),
            "note": "read + write bytes of a 1 GiB device copy, the better of a plain streaming "
                    "copy kernel and torch's copy; 256 MiB pinned-host DMA each way"}


def _probe_lib():
    """The measurement library built beside the hot-path library."""
    import ctypes
    from serving_memory_tier_amd import build
    if not os.path.exists(build.PROBE_LIB):
        raise RuntimeError(f"{build.PROBE_LIB} is missing; build with __graft_entry__.build()")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.hs_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hs_probe_copy.restype = ctypes.c_int
    return lib


def touch_cost(wl, dev, hev, stream: int, i: int, n: int, busy=None):
    """hs_page_touch on step i's lists: n launches back to back between one
    pair of HIP events on the launch stream; algorithmic bytes: every list
    entry read once, one 4-byte word written per distinct page touched."""
    import numpy as np
    import torch

    from serving_memory_tier_amd import hs_page_touch
    use = torch.zeros((wl.R, wl.max_pages), dtype=torch.int32, device="cuda")
    E = wl.NG * wl.P * wl.K
    # a launch takes a few microseconds, less than an event pair's own cost
    # and less than the host's enqueue of one call: the n launches are
    # captured once and the graph's replay is timed between one event pair
    cap = torch.cuda.Stream()
    hev.begin_capture(cap.cuda_stream)
    try:
        for j in range(n):
            hs_page_touch(dev.layout, dev.batches[i], dev.topk[i], E, wl.steps[i].stamp, use,
                          cap.cuda_stream)
    finally:
        hev.end_capture(cap.cuda_stream)
    a, b = hev.new_event(system_fence=False), hev.new_event(system_fence=False)
    hev.launch(stream)                    # warm replay
    torch.cuda.synchronize()
    if busy is not None:
        busy.fill()
    hev.record(a, stream)
    hev.launch(stream)
    hev.record(b, stream)
    torch.cuda.synchronize()
    hev.destroy_graph()
    us = 1e3 * hev.elapsed_ms(a, b) / n
    pages = int((use != 0).sum().item())
    nbytes = wl.R * E * 4 + pages * 4
    return {"us": round(us, 2), "hbm_bytes": nbytes, "hbm_gbps": round(nbytes / us / 1e3, 1),
            "pages_touched": pages}


def policy_cost(wl, dev, n: int = 20):
    """Host cost of one residency-policy step at this batch's shape: every
    request admitted with its complete pages on host (resident prefix for
    every other request), then n steps of one appended token each, with
    coldness from the GPU's per-page stamps (hs_page_touch) or from the lists
    themselves.  Milliseconds per step, median; the policy never runs on the
    decode path, this is what it costs between steps."""
    import numpy as np
    import torch

    from serving_memory_tier_amd import hs_page_touch
    from serving_memory_tier_amd import policy as pol
    R, E = wl.R, wl.NG * wl.P * wl.K
    ctx = wl.ctx0.astype(np.int64).copy()
    pages0 = (ctx + PAGE - 1) // PAGE
    max_pages = int(pages0.max()) + n + 2
    need = int(pages0[::2].sum()) + (R - R // 2) * (4 + wl.C // PAGE)
    host_total = int((ctx // PAGE).sum())
    out = {}
    for form in ("page_stamps", "lists"):
        p = pol.Policy(PAGE, need + 8, host_total + R * (n + 2), R, max_pages, wl.C // PAGE, 4)
        base = R * (n + 2)
        for r in range(R):
            hb = np.arange(base, base + int(ctx[r]) // PAGE, dtype=np.int32)
            base += hb.size
            p.admit(r, int(ctx[r]), hb, r % 2 == 0)
        use = torch.zeros((R, max_pages), dtype=torch.int32, device="cuda")
        c_dev = torch.from_numpy(ctx.astype(np.int32)).cuda()
        from serving_memory_tier_amd._lib import HsBatch
        batch = HsBatch(R, max_pages, None, None, None, None, c_dev.data_ptr(), None, None, None)
        times = []
        c = ctx.copy()
        for s in range(n):
            i = s % len(wl.steps)
            topk = dev.topk[i]
            hs_page_touch(dev.layout, batch, topk, E, s + 1, use)
            torch.cuda.synchronize()
            c = c + 1
            if form == "page_stamps":
                u = use.cpu().numpy().view(np.uint32)
                t0 = time.perf_counter()
                p.step_pages(np.arange(R), c, u)
            else:
                lists = topk.cpu().numpy().reshape(R, -1)
                t0 = time.perf_counter()
                p.step(s + 2, np.arange(R), c, lists)
            times.append(time.perf_counter() - t0)
            c_dev.copy_(torch.from_numpy(c.astype(np.int32)))
        out[form + "_ms"] = round(1e3 * float(np.median(times)), 3)
        p.close()
    out["note"] = ("host ms per policy step (median of %d) at this batch's shape; the GPU's "
                   "per-page stamps (hs_page_touch) replace a scan of every list entry" % n)
    return out


def _oracle_run(wl, budget_s: float, threads: int):
    """The oracle on the workload's steps (all requests, resolve + gather +
    offload), passes over them from the initial state until the time budget is
    used: (steps done, passes begun, seconds).  With threads > 1 each step's
    requests are cut into that many contiguous blocks resolved at once
    (request-layers are independent, and the oracle's C++ call runs without
    the interpreter lock).  Only the oracle's calls are timed."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle

    cuts = np.linspace(0, wl.R, threads + 1).astype(int)
    blocks = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    pool_ex = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
    pool = np.zeros((wl.L, wl.pool_rows, ROW), dtype=np.uint8)
    host = np.zeros((wl.L, wl.host_rows, ROW), dtype=np.uint8)
    wl.fill_device_pool(torch.from_numpy(pool))
    wl.fill_host_pool(torch.from_numpy(host))
    done, spent, passes = 0, 0.0, 0
    try:
        while spent < budget_s:
            # each pass from the initial tables and hot-buffer state; the pools
            # keep the bytes earlier passes wrote, which decide no step's work
            passes += 1
            bt, hbt = wl.block_table.copy(), wl.host_block_table.copy()
            tok = np.full((wl.R, wl.L, wl.C), -1, np.int32)
            stp = np.zeros((wl.R, wl.L, wl.C), np.uint32)
            for s in wl.steps:
                for r, p, v in s.hbt_set:
                    hbt[r, p] = v
                for r, p, v in s.bt_set:
                    bt[r, p] = v
                topk = np.ascontiguousarray(s.topk)
                t = time.perf_counter()
                if pool_ex is None:
                    oracle.resolve(pool, host, bt, hbt, s.ctx, wl.hot_blocks, tok, stp, topk,
                                   s.stamp, True)
                else:
                    def part(ab):
                        a, b = ab
                        return oracle.resolve(pool, host, bt[a:b], hbt[a:b], s.ctx[a:b],
                                              wl.hot_blocks[a:b], tok[a:b], stp[a:b], topk[a:b],
                                              s.stamp, True)
                    list(pool_ex.map(part, blocks))
                if s.offload.shape[0]:
                    oracle.offload(pool, host, s.offload)
                spent += time.perf_counter() - t
                done += 1
                if spent >= budget_s:
                    break
    finally:
        if pool_ex is not None:
            pool_ex.shutdown()
    return done, passes, spent


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, single-threaded, on the same workload (all
    requests, resolve + gather), passes over its steps until the time budget
    is used; then the same with one thread per host core (at most 16) over
    blocks of requests."""
    done, passes, spent = _oracle_run(wl, budget_s, 1)
    rows = done * wl.R * wl.L * wl.P * wl.K
    res = {"value": round(rows / spent), "unit": "rows/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} steps of {wl.name} ({passes} pass(es) over "
                     f"its {len(wl.steps)} steps, each from the initial tables and hot-buffer state; "
                     f"{wl.R} requests x {wl.L} layers, resolve + "
                     f"gather + offload), {spent:.1f}s single-threaded"}
    threads = max(1, min(16, os.cpu_count() or 1, wl.R))
    if threads > 1:
        d2, p2, s2 = _oracle_run(wl, budget_s, threads)
        res["multi_thread"] = {"value": round(d2 * wl.R * wl.L * wl.P * wl.K / s2),
                               "unit": "rows/s", "cores": threads,
                               "sample": f"{d2} steps ({p2} pass(es)), {s2:.1f}s, requests "
                                         f"split into {threads} blocks"}
    return res


if __name__ == "__main__":
    main()
