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
launch stream, algorithmic bytes per launch), the achieved HBM and host-link
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
HOST_LINK_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction
ROW = 656
PAGE = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="mixed_decode",
                    choices=["mixed_decode", "no_residency", "mixed_state", "multi_layer"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hit-replays", type=int, default=50)
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying a captured graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain 256 MiB device copy (counter calibration runs)")
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
    return hs_gen.multi_layer(turns=n_steps)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when it was taken on another workload or on other kernel sources."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters_decide_move_mixed_decode.md")
    if workload != "mixed_decode" or not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in ("resolve.hip", "copy.hip", "hs_internal.h"):
        with open(os.path.join(ROOT, "serving_memory_tier_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    v = fields.get(f"{kernel}_traffic_bytes_per_launch")
    return int(v) if v else None


def decide_hbm_bytes(wl, stats_sum, n_launches):
    """Algorithmic HBM bytes of the decision kernel per launch.

    Per request-layer: the slot tokens and stamps are read once (8 B/slot).
    Per entry: the index (4 B), its block-table entry (4 B), its row (4 B).
    Per hit: the refreshed stamp (4 B).  Per miss: the host-table entry (4 B)
    and the slot's new token and stamp (8 B).
    """
    R, L, N = wl.R, wl.L, wl.P * wl.K
    hits, misses = stats_sum[1], stats_sum[2]
    return R * L * wl.C * 8 + R * L * N * 12 + (hits * 4 + misses * 12) / n_launches


def move_hbm_bytes(wl, stats_sum, n_launches):
    """Algorithmic HBM bytes of the row mover per launch: every entry reads its
    row code (4 B) and writes its 656-B output row; every resident or hit entry
    reads its 656-B row from the pool; every miss writes its row into the hot
    slot (656 B) and its final row id (4 B) -- its read comes over the host link."""
    R, L, N = wl.R, wl.L, wl.P * wl.K
    entries = R * L * N
    misses = stats_sum[2] / n_launches
    return entries * (4 + ROW) + (entries - misses) * ROW + misses * (ROW + 4)


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
    t_gen = time.time()
    wl = build_workload(args.workload, W + K + KE)
    print(f"[bench] workload {wl.name}: R={wl.R} L={wl.L} P={wl.P} K={wl.K} C={wl.C} "
          f"steps={len(wl.steps)} generated in {time.time() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    dev = DeviceRun(wl)
    dev.upload_steps()
    n_steps = len(wl.steps)
    N = wl.P * wl.K
    entries = wl.R * wl.L * N
    dev.stage_steps()
    stats_all = torch.zeros((n_steps, wl.R, wl.L, 8), dtype=torch.int32, device="cuda")
    hev = HipRuntime()

    def step(i, sp, ev=None):
        dev.launch_step(i, hev, sp, stats=stats_all[i], events=ev)

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

    # per-kernel durations: the next KE steps launched one by one, HIP events
    # on the launch stream around every kernel
    events = [[hev.new_event() for _ in range(4)] for _ in range(KE)]
    for j in range(KE):
        step(W + K + j, sp0, events[j])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    dec_ms = [hev.elapsed_ms(events[j][0], events[j][1]) for j in range(KE)]
    mov_ms = [hev.elapsed_ms(events[j][1], events[j][2]) for j in range(KE)]
    off = [(j, hev.elapsed_ms(events[j][2], events[j][3])) for j in range(KE)
           if wl.steps[W + K + j].offload.shape[0]]
    st = stats_all[W + K:W + K + KE].sum(dim=(0, 1, 2)).cpu().numpy().astype(np.int64)
    st_all = stats_all[W:W + K].sum(dim=(0, 1, 2)).cpu().numpy().astype(np.int64)
    dec_us = 1e3 * float(np.mean(dec_ms))
    mov_us = 1e3 * float(np.mean(mov_ms))
    value = entries * K / wall

    dec_bytes = decide_hbm_bytes(wl, st, KE)
    mov_bytes = move_hbm_bytes(wl, st, KE)
    host_bytes = st[2] * ROW / KE
    kernels = {
        "decide": {"us": round(dec_us, 2), "hbm_bytes": int(dec_bytes),
                   "hbm_gbps": round(dec_bytes / dec_us / 1e3, 1)},
        "move": {"us": round(mov_us, 2), "hbm_bytes": int(mov_bytes),
                 "hbm_gbps": round(mov_bytes / mov_us / 1e3, 1),
                 "host_link_bytes": int(host_bytes),
                 "host_link_gbps": round(host_bytes / mov_us / 1e3, 2)},
    }
    if off:
        page_layers = [wl.steps[W + K + j].offload.shape[0] * wl.L for j, _ in off]
        off_us = 1e3 * float(np.mean([ms for _, ms in off]))
        off_bytes = float(np.mean(page_layers)) * PAGE * ROW
        kernels["offload"] = {"us": round(off_us, 2), "launches": len(off),
                              "host_link_bytes": int(off_bytes),
                              "host_link_gbps": round(off_bytes / off_us / 1e3, 2)}

    # the hit-replay path: the last step's lists again with the same stamp --
    # every non-resident token hits, no host traffic, HBM-bound
    last = W + K + KE - 1
    rep = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.hit_replays)]
    rep_stats = torch.zeros((wl.R, wl.L, 8), dtype=torch.int32, device="cuda")
    for j in range(args.hit_replays):
        rep[j][0].record(stream)
        hs.hs_resolve_decide(dev.layout, dev.batches[last], dev.topk[last], wl.P, wl.K,
                             wl.steps[last].stamp, dev.rows, rep_stats, sp)
        rep[j][1].record(stream)
        hs.hs_resolve_move(dev.layout, dev.batches[last], dev.topk[last], wl.P, wl.K, dev.rows,
                           dev.out, sp)
        rep[j][2].record(stream)
    torch.cuda.synchronize()
    rs = rep_stats.sum(dim=(0, 1)).cpu().numpy()
    rd_us = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in rep]))
    rm_us = 1e3 * float(np.mean([e[1].elapsed_time(e[2]) for e in rep]))
    rep_bytes = decide_hbm_bytes(wl, rs, 1) + move_hbm_bytes(wl, rs, 1)
    hit_replay = {"decide_us": round(rd_us, 2), "move_us": round(rm_us, 2),
                  "misses": int(rs[2]),
                  "rows_per_s": round(entries / ((rd_us + rm_us) * 1e-6)),
                  "hbm_gbps": round(rep_bytes / (rd_us + rm_us) / 1e3, 1),
                  "hbm_frac": round(rep_bytes / (rd_us + rm_us) / 1e3 / HBM_PEAK_GBPS, 4),
                  "move_hbm_gbps": round(move_hbm_bytes(wl, rs, 1) / rm_us / 1e3, 1)}

    # the dominant kernel of a step and the resource that bounds it: the
    # mover is bound by the host link when it carries misses (its HBM bytes
    # would take a fraction of the time at HBM speed), by HBM otherwise
    if mov_us >= dec_us:
        host_t = host_bytes / (HOST_LINK_PEAK_GBPS * 1e3)
        hbm_t = mov_bytes / (HBM_PEAK_GBPS * 1e3)
        if host_t >= hbm_t:
            ach = host_bytes / mov_us / 1e3
            roofline = {"kernel": "move", "bound": "host_link", "achieved": round(ach, 2),
                        "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(ach / HOST_LINK_PEAK_GBPS, 4), "traffic": None}
        else:
            ach = mov_bytes / mov_us / 1e3
            roofline = {"kernel": "move", "bound": "hbm", "achieved": round(ach, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None}
    else:
        ach = dec_bytes / dec_us / 1e3
        roofline = {"kernel": "decide", "bound": "hbm", "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "traffic": None}
    roofline["traffic"] = measured_traffic(roofline["kernel"], wl.name)
    # whole steps of the timed region: algorithmic bytes per step / step time
    step_hbm_k = decide_hbm_bytes(wl, st_all, K) + move_hbm_bytes(wl, st_all, K)
    host_k = st_all[2] * ROW / K
    line = {
        "metric": METRIC, "value": round(value), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(1e3 * wall / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.R, "layers": wl.L, "positions": wl.P,
                   "top_k": wl.K, "hot_capacity": wl.C, "context": int(wl.ctx0.max()),
                   "row_bytes": ROW, "page_size": PAGE, "launch": launch},
        "hbm": {"achieved": round(step_hbm_k / (wall / K) / 1e9, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(step_hbm_k / (wall / K) / 1e9 / HBM_PEAK_GBPS, 4)},
        "host_link": {"achieved": round(host_k / (wall / K) / 1e9, 2),
                      "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(host_k / (wall / K) / 1e9 / HOST_LINK_PEAK_GBPS, 4)},
        "per_step": {"hits": round(st_all[1] / K, 1), "misses": round(st_all[2] / K, 1),
                     "resident": round(st_all[0] / K, 1)},
        "kernels": kernels,
        "kernel_timing": f"HIP events around each kernel over {KE} eagerly launched steps "
                         f"following the timed ones",
        "hit_replay": hit_replay,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    hev.destroy_graph()
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


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, single-threaded, on the first steps of the same
    workload (all requests, resolve + gather), until the time budget is used."""
    import numpy as np
    import torch

    import oracle

    pool = np.zeros((wl.L, wl.pool_rows, ROW), dtype=np.uint8)
    host = np.zeros((wl.L, wl.host_rows, ROW), dtype=np.uint8)
    wl.fill_device_pool(torch.from_numpy(pool))
    wl.fill_host_pool(torch.from_numpy(host))
    bt, hbt = wl.block_table.copy(), wl.host_block_table.copy()
    tok = np.full((wl.R, wl.L, wl.C), -1, np.int32)
    stp = np.zeros((wl.R, wl.L, wl.C), np.uint32)
    done, spent = 0, 0.0
    for s in wl.steps:
        for r, p, v in s.hbt_set:
            hbt[r, p] = v
        for r, p, v in s.bt_set:
            bt[r, p] = v
        t = time.perf_counter()
        oracle.resolve(pool, host, bt, hbt, s.ctx, wl.hot_blocks, tok, stp,
                       np.ascontiguousarray(s.topk), s.stamp, True)
        if s.offload.shape[0]:
            oracle.offload(pool, host, s.offload)
        spent += time.perf_counter() - t
        done += 1
        if spent >= budget_s:
            break
    rows = done * wl.R * wl.L * wl.P * wl.K
    return {"value": round(rows / spent), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} steps of {wl.name} ({wl.R} requests x {wl.L} layers, "
                      f"resolve + gather + offload), {spent:.1f}s single-threaded"}


if __name__ == "__main__":
    main()
