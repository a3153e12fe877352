"""The resolver's stages driven from Python, for tests that check each path of
the library against the oracle:

  call    -- hs_resolve / hs_plan_replay (the overlapped form inside the
             library when there is a gather output);
  fused   -- the same as stages: hs_resolve_decide with the gather output (the
             resolver's and the early fill's workgroups in one launch), then
             hs_resolve_commit;
  serial  -- hs_resolve_decide, then hs_resolve_move (host copies in the mover);
  staged  -- the overlapped form scheduled by the caller: hs_resolve_decide on a
             second stream, hs_resolve_fetch (the early fill of every output
             row) on the first, a join, then hs_resolve_commit;
  in_place -- hs_resolve_in_place: no gathered rows (``out`` is only staging
             for the misses' host rows), for consumers that read rows by id.
"""

from __future__ import annotations

import torch

import serving_memory_tier_amd as hs

MODES = ("call", "fused", "serial", "staged", "in_place")


def run(mode, layout, batch, topk, P, K, stamp, rows, out, stats, pairs=None, n_pairs=0,
        aux=None):
    """One resolve (plus the optional offload) on torch's current stream."""
    if mode == "call":
        if P == 1 and n_pairs == 0:
            hs.hs_resolve(layout, batch, topk, K, stamp, rows, out, stats)
        else:
            hs.hs_plan_replay(layout, batch, topk, P, K, stamp, rows, out, stats, pairs, n_pairs)
        return
    if mode == "in_place":
        assert out is not None, "the in-place form stages misses in a buffer of the output's size"
        hs.hs_resolve_in_place(layout, batch, topk, P, K, stamp, rows, out, stats, pairs, n_pairs)
        return
    main = torch.cuda.current_stream()
    if mode == "serial":
        hs.hs_resolve_decide(layout, batch, topk, P, K, stamp, rows, None, stats)
        hs.hs_resolve_move(layout, batch, topk, P, K, rows, out)
    elif mode == "fused":
        assert out is not None, "the fused form needs a gather output"
        hs.hs_resolve_decide(layout, batch, topk, P, K, stamp, rows, out, stats)
        hs.hs_resolve_commit(layout, batch, topk, P, K, rows, out)
    elif mode == "staged":
        assert out is not None, "the staged form needs a gather output"
        aux = aux or torch.cuda.Stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        aux.wait_event(fork)
        hs.hs_resolve_decide(layout, batch, topk, P, K, stamp, rows, None, stats, aux)
        join.record(aux)
        hs.hs_resolve_fetch(layout, batch, topk, P, K, out)
        main.wait_event(join)
        hs.hs_resolve_commit(layout, batch, topk, P, K, rows, out)
    else:
        raise ValueError(mode)
    if n_pairs:
        hs.hs_offload_prefix_pages(layout, batch.kv_pool, batch.host_pool, pairs, n_pairs)
