"""GPU parity of hs_sparse_mla_decode (sparse MLA decode reading the resolved
rows in place by row id) with the float64 oracle, within the tolerance the
arithmetic fixes: keys and values are exact (E4M3 values are bfloat16
values, scales applied in float32), products accumulate in float32, and the
roundings that matter are of p_j * scale to bfloat16 for the value products,
a relative 2^-9 on each term, and, where the keys are split across
workgroups, of each split's normalised output to half precision, a relative
2^-11 -- so |out - out_ref| <= (2^-9 + 2^-11) * max_j |v_j|; the test allows
2^-8 * max_j |v_j| + 1e-6, and 1e-4 on lse."""

from __future__ import annotations

import math
import os
import zlib

import numpy as np
import pytest
import torch

from oracle import sparse_mla as sm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import serving_memory_tier_amd as hs
    if not os.path.exists(hs.LIB_PATH):
        from serving_memory_tier_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hs.lib()


def make_pool(rs, n_rows, max_exp=8, scale=(0.05, 0.3)):
    """Random FP8 rows: latent bytes of exponent field <= max_exp (no NaN),
    scales in the given range, rope bf16 of a unit normal."""
    sign = rs.integers(0, 2, size=(n_rows, 512)) << 7
    e = rs.integers(0, max_exp + 1, size=(n_rows, 512)) << 3
    m = rs.integers(0, 8, size=(n_rows, 512))
    pool = np.zeros((n_rows, 656), np.uint8)
    pool[:, :512] = (sign | e | m).astype(np.uint8)
    pool[:, 512:528] = rs.uniform(*scale, size=(n_rows, 4)).astype("<f4").view(np.uint8)
    rope = (rs.standard_normal((n_rows, 64)).astype(np.float32).view(np.uint32) >> 16)
    pool[:, 528:] = rope.astype("<u2").view(np.uint8)
    return pool


def make_q(rs, T, H, mult=1.0):
    return ((rs.standard_normal((T, H, 576)) * mult).astype(np.float32).view(np.uint32)
            >> 16).astype(np.uint16)


def run_gpu(pool, ids, q, sm_scale, kv_rows=None):
    import serving_memory_tier_amd as hs
    T, K = ids.shape
    H = q.shape[1]
    # page size 1: any row count is a whole number of pages
    lay = hs.layout_of(1, 656, 1, 64, pool.shape[0] if kv_rows is None else kv_rows, 0)
    gp = torch.from_numpy(pool).cuda()
    gi = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
    gq = torch.from_numpy(q.view(np.int16)).cuda()
    out = torch.full((T, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    wsb = hs.hs_sparse_mla_workspace_bytes(T, H, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    print(f"[attend] T={T} H={H} K={K} pool_rows={pool.shape[0]} workspace={wsb}", flush=True)
    hs.hs_sparse_mla_decode(lay, gp, gi, T, K, gq, H, sm_scale, out, lse, ws, wsb)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(pool, ids, q, sm_scale):
    out, lse = run_gpu(pool, ids, q, sm_scale)
    ref_out, ref_lse = sm.sparse_mla_decode(pool, ids, q, sm_scale)
    _, v_all = sm.decode_rows(pool)
    for t in range(ids.shape[0]):
        sel = ids[t][(ids[t] >= 0) & (ids[t] < pool.shape[0])]
        if sel.size == 0:
            assert (out[t] == 0).all() and np.isneginf(lse[t]).all()
            continue
        vmax = np.abs(v_all[sel]).max()
        err = np.abs(out[t] - ref_out[t]).max()
        assert err <= 2.0 ** -8 * vmax + 1e-6, (t, err, vmax)
        assert np.abs(lse[t] - ref_lse[t]).max() <= 1e-4, t
    return out, lse


CASES = {  # name: (T, H, K, pool rows, q multiplier, invalid share)
    "single_row": (2, 16, 1, 8, 1.0, 0.0),
    "ragged_300": (3, 32, 300, 900, 1.0, 0.1),
    "heads_48_k2048": (1, 48, 2048, 3000, 1.0, 0.05),
    "peaky_scores": (2, 64, 777, 2000, 6.0, 0.02),
    "heads_128_k512": (4, 128, 512, 1500, 1.0, 0.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_mla_matches_oracle(name):
    T, H, K, n, mult, bad = CASES[name]
    rs = np.random.default_rng(zlib.crc32(name.encode()))
    pool = make_pool(rs, n)
    q = make_q(rs, T, H, mult)
    ids = rs.integers(0, n, size=(T, K)).astype(np.int32)
    ids[rs.random((T, K)) < bad] = rs.choice([-1, -2, -3, n, n + 5], size=1)[0]
    if K > 4:
        ids[0, 1] = ids[0, 0]                       # a duplicate counts twice
    check(pool, ids, q, 1.0 / math.sqrt(576))


def _sweep_case(seed):
    """Shape and value ranges of attention sweep case ``seed``: tokens, heads
    (multiples of 16), selected rows, pool size, query scale, the share of
    unselected or out-of-range ids, and the latent values' largest exponent."""
    rs = np.random.default_rng(7000 + seed)
    T = int(rs.integers(1, 7))
    H = 16 * int(rs.integers(1, 9))
    K = int(rs.integers(1, 3001))
    while T > 1 and T * H * K > 1_500_000:
        T -= 1
    n = int(rs.integers(K // 2 + 1, 4001))
    mult = float(rs.choice([0.5, 1.0, 3.0, 8.0]))
    bad = float(rs.choice([0.0, 0.02, 0.2, 0.9]))
    max_exp = int(rs.choice([6, 8, 14]))
    return rs, T, H, K, n, mult, bad, max_exp


@pytest.mark.parametrize("seed", list(range(16)))
def test_sparse_mla_sweep(seed):
    """Random shapes: 1-6 tokens, 16-128 heads, 1-3000 selected rows (so 1 to
    many key splits and ragged last blocks), query scales up to 8 (peaky
    scores), up to 90 % of the ids unselected or out of range."""
    rs, T, H, K, n, mult, bad, max_exp = _sweep_case(seed)
    pool = make_pool(rs, n, max_exp=max_exp)
    q = make_q(rs, T, H, mult)
    ids = rs.integers(0, n, size=(T, K)).astype(np.int32)
    m = rs.random((T, K)) < bad
    ids[m] = rs.choice(np.array([-1, -2, -3, n, n + 5], np.int32), size=int(m.sum()))
    check(pool, ids, q, 1.0 / math.sqrt(576))


def test_nothing_selected_and_empty_lists():
    rs = np.random.default_rng(7)
    pool = make_pool(rs, 10)
    q = make_q(rs, 3, 16)
    ids = np.array([[-1, -2, -3, 10, 11], [0, -1, -1, -1, -1], [-1] * 5], np.int32)
    check(pool, ids, q, 0.05)
    out, lse = run_gpu(pool, np.zeros((2, 0), np.int32), make_q(rs, 2, 16), 0.05)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_decode_shape_sampled():
    """The decode shape: 32 tokens x 128 heads x 2048 selected rows."""
    rs = np.random.default_rng(11)
    n = 20000
    pool = make_pool(rs, n)
    q = make_q(rs, 32, 128)
    ids = rs.integers(0, n, size=(32, 2048)).astype(np.int32)
    ids[:, -5:] = -1
    check(pool, ids, q, 1.0 / math.sqrt(576))


def _sanitize(t: torch.Tensor) -> None:
    """Make a pool of synthetic bytes a pool of valid FP8 MLA rows, in place
    and the same way everywhere (so copies between pools stay copies):
    latent bytes lose bit 6 (|value| < 2, no NaN), the scales become 1/16,
    the rope values lose their exponent's top bits (|value| < 2)."""
    rows = t.view(-1, 656)
    rows[:, :512] &= 0xBF
    rows[:, 512:528] = torch.tensor(list(np.float32(1.0 / 16).tobytes()) * 4, dtype=torch.uint8,
                                    device=t.device)
    rows[:, 529:656:2] &= 0xBF


def test_consumer_reads_in_place_what_the_gather_delivers():
    """A decode step consumed two ways gives bit-identical attention: the
    resolver in place (hs_resolve_in_place, only the misses staged) then the
    kernel reading the pool by row id, or the resolver with its gathered
    output then the kernel reading the gathered rows; and both match the
    oracle on the step's rows."""
    import serving_memory_tier_amd as hs
    import hs_gen
    from serving_memory_tier_amd.runner import DeviceRun
    wl = hs_gen.mixed_decode(steps=4)
    T, K, H = wl.R, wl.K, 32
    runs = []
    for mode in ("in_place", "gathered"):
        dev = DeviceRun(wl)
        dev.upload_steps()
        _sanitize(dev.pool)
        _sanitize(dev.host)
        runs.append(dev)
    rs = np.random.default_rng(3)
    q = torch.from_numpy(make_q(rs, T, H).view(np.int16)).cuda()
    iota = torch.arange(T * K, dtype=torch.int32, device="cuda").view(T, K)
    wsb = hs.hs_sparse_mla_workspace_bytes(T, H, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    lay_pool = hs.layout_of(64, 656, 1, 64, wl.pool_rows, 0)
    lay_out = hs.layout_of(1, 656, 1, 64, T * K, 0)
    scale = 1.0 / math.sqrt(576)
    try:
        for i, step in enumerate(wl.steps):
            res = []
            for mode, dev in zip(("in_place", "gathered"), runs):
                print(f"[attend] consumer {mode} step {i}", flush=True)
                dev.pre(i)
                out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
                lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
                n = step.offload.shape[0]
                if mode == "in_place":
                    hs.hs_resolve_in_place(dev.layout, dev.batch, dev.topk[i], 1, K, step.stamp,
                                           dev.rows, dev.out, dev.stats,
                                           dev.pairs[i] if n else None, n)
                    hs.hs_sparse_mla_decode(lay_pool, dev.pool, dev.rows, T, K, q, H, scale, out,
                                            lse, ws, wsb)
                else:
                    dev.plan_step(i)
                    hs.hs_sparse_mla_decode(lay_out, dev.out, iota, T, K, q, H, scale, out, lse,
                                            ws, wsb)
                torch.cuda.synchronize()
                res.append((out.cpu().numpy(), lse.cpu().numpy(), dev.rows.cpu().numpy()))
            assert np.array_equal(res[0][2], res[1][2]), f"row ids, step {i}"
            assert np.array_equal(res[0][0].view(np.int32), res[1][0].view(np.int32)), i
            assert np.array_equal(res[0][1].view(np.int32), res[1][1].view(np.int32)), i
            # the oracle on three requests' rows, from the pool as it stands
            pool = runs[0].pool[0].cpu().numpy()
            ids = res[0][2].reshape(T, K)
            qn = q.cpu().numpy().view(np.uint16)
            for r in (0, 7, 31):
                ref_o, ref_l = sm.sparse_mla_decode(pool, ids[r:r + 1], qn[r:r + 1], scale)
                sel = ids[r][(ids[r] >= 0) & (ids[r] < pool.shape[0])]
                vmax = np.abs(sm.decode_rows(pool[sel])[1]).max()
                assert np.abs(res[0][0][r] - ref_o[0]).max() <= 2.0 ** -8 * vmax + 1e-6
                assert np.abs(res[0][1][r] - ref_l[0]).max() <= 1e-4
    finally:
        for dev in runs:
            dev.close()
