"""Host logic of the workload runner (no GPU): the scheduler's table updates
of a step, cut into runs that one copy each writes."""

from __future__ import annotations

import numpy as np

from serving_memory_tier_amd.runner import update_runs


def _apply_runs(table: np.ndarray, arr: np.ndarray) -> np.ndarray:
    R, max_pages = table.shape
    flat = table.reshape(-1)
    for r, p, along_pages, vals in update_runs(arr):
        stride = 1 if along_pages else max_pages
        idx = r * max_pages + p + stride * np.arange(vals.shape[0])
        # a run stays inside one request's row or one page's column
        if along_pages:
            assert p + vals.shape[0] <= max_pages
        else:
            assert r + vals.shape[0] <= R
        flat[idx] = vals
    return table


def test_runs_write_every_update_once():
    rng = np.random.default_rng(5)
    R, max_pages = 12, 40
    for _ in range(300):
        n = int(rng.integers(0, 80))
        cells = rng.choice(R * max_pages, size=n, replace=False)
        vals = rng.integers(-1, 100000, size=n)
        arr = np.stack([cells // max_pages, cells % max_pages, vals], axis=1).astype(np.int64)
        direct = np.full((R, max_pages), 7, np.int32)
        for r, p, v in arr:
            direct[r, p] = v
        runs = update_runs(arr)
        assert sum(v.shape[0] for *_, v in runs) == n
        assert np.array_equal(_apply_runs(np.full((R, max_pages), 7, np.int32), arr), direct)


def test_a_completed_page_is_one_strided_copy():
    # every request's host-table entry for page 17
    arr = np.array([[r, 17, 1000 + r] for r in range(32)], dtype=np.int64)
    runs = update_runs(arr)
    assert len(runs) == 1
    r, p, along_pages, vals = runs[0]
    assert (r, p, along_pages) == (0, 17, False)
    assert vals.tolist() == [1000 + r for r in range(32)]


def test_consecutive_pages_of_a_request_are_one_contiguous_copy():
    arr = np.array([[3, p, -1] for p in range(20, 31)] + [[5, 2, 9]], dtype=np.int64)
    runs = update_runs(arr)
    assert len(runs) == 2
    assert (runs[0][0], runs[0][1], runs[0][2], runs[0][3].shape[0]) == (3, 20, True, 11)


def test_no_updates_no_runs():
    assert update_runs(np.zeros((0, 3), dtype=np.int64)) == []
