"""Pins of the sparse MLA decode oracle (oracle/sparse_mla.py), on the CPU:
FP8 E4M3 and bfloat16 values the formats fix, a hand-built row, closed forms
of the attention (one row, equal scores, duplicates, nothing selected),
invariances, and a brute-force restatement with scalar loops on tiny inputs.
Planted mistakes in copies of the oracle's steps must fail these pins."""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import sparse_mla as sm


def _row(lat_bytes, scales, rope_bits):
    r = np.zeros(sm.ROW_BYTES, np.uint8)
    r[:512] = lat_bytes
    r[512:528] = np.asarray(scales, "<f4").view(np.uint8)
    r[528:] = np.asarray(rope_bits, "<u2").view(np.uint8)
    return r


def test_fp8_values_fixed_by_the_format():
    v = sm.fp8_e4m3_value
    assert v(0x38) == 1.0 and v(0x30) == 0.5 and v(0x39) == 1.125 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite
    assert v(0x08) == 2.0 ** -6                             # smallest normal
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    finite = [v(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(finite, finite[1:]))   # monotone over the positives
    assert all(v(b | 0x80) == -v(b) for b in range(0x7F))


def test_bf16_values():
    f = sm.bf16_to_float(np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x4049], np.uint16))
    assert f[:4].tolist() == [1.0, -2.0, 0.25, 0.0]
    assert abs(f[4] - 3.140625) < 1e-12


def test_decode_hand_built_row():
    lat = np.full(512, 0x38, np.uint8)                      # every latent value 1.0
    lat[5] = 0x40                                           # 2.0
    lat[300] = 0xB0                                         # -0.5
    rope = np.full(64, 0x3F80, np.uint16)
    rope[63] = 0xC000
    k, v = sm.decode_rows(_row(lat, [2.0, 0.5, 4.0, -1.0], rope)[None])
    exp = np.concatenate([np.full(128, 2.0), np.full(128, 0.5), np.full(128, 4.0),
                          np.full(128, -1.0)])
    exp[5] = 4.0
    exp[300] = -2.0                                         # tile 2: -0.5 * 4
    assert np.array_equal(v[0], exp)
    assert np.array_equal(k[0, :512], exp)
    assert np.array_equal(k[0, 512:], np.r_[np.ones(63), -2.0])


def _pool(rs, n):
    pool = np.zeros((n, sm.ROW_BYTES), np.uint8)
    for i in range(n):
        lat = rs.integers(0, 256, 512).astype(np.uint8)
        lat[(lat & 0x7F) == 0x7F] = 0x38                    # no NaN bytes
        sc = rs.uniform(0.01, 0.05, 4)
        rope = (rs.standard_normal(64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        pool[i] = _row(lat, sc, rope)
    return pool


def _q(rs, T, H):
    return (rs.standard_normal((T, H, 576)).astype(np.float32).view(np.uint32)
            >> 16).astype(np.uint16)


def test_one_selected_row_is_its_value():
    rs = np.random.default_rng(1)
    pool, q = _pool(rs, 6), _q(rs, 1, 3)
    out, lse = sm.sparse_mla_decode(pool, np.array([[4, -1, -3, 6, -2]], np.int32), q, 0.125)
    k, v = sm.decode_rows(pool[4:5])
    assert np.allclose(out[0], np.repeat(v, 3, axis=0), rtol=0, atol=1e-12)
    assert np.allclose(lse[0], 0.125 * (sm.bf16_to_float(q[0]) @ k[0]), rtol=0, atol=1e-12)


def test_equal_scores_average_and_duplicates_weigh_double():
    lat = [np.full(512, b, np.uint8) for b in (0x38, 0x40)]    # rows of 1.0 and 2.0
    pool = np.stack([_row(lat[0], [1, 1, 1, 1], np.zeros(64)),
                     _row(lat[1], [1, 1, 1, 1], np.zeros(64))])
    q = np.zeros((1, 1, 576), np.uint16)                       # zero query: equal scores
    out, lse = sm.sparse_mla_decode(pool, np.array([[0, 1]], np.int32), q, 1.0)
    assert np.allclose(out, 1.5, rtol=0, atol=1e-12) and np.isclose(lse[0, 0], math.log(2))
    out, lse = sm.sparse_mla_decode(pool, np.array([[0, 0, 1]], np.int32), q, 1.0)
    assert np.allclose(out, 4.0 / 3.0, rtol=0, atol=1e-12) and np.isclose(lse[0, 0], math.log(3))


def test_nothing_selected():
    rs = np.random.default_rng(2)
    pool, q = _pool(rs, 3), _q(rs, 2, 2)
    out, lse = sm.sparse_mla_decode(pool, np.array([[-1, -2, 3, 99], [0, -1, -1, -1]], np.int32),
                                    q, 0.1)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(lse[1]).all()


def test_permutation_invariance():
    rs = np.random.default_rng(3)
    pool, q = _pool(rs, 40), _q(rs, 2, 4)
    ids = rs.integers(-2, 40, size=(2, 33)).astype(np.int32)
    a = sm.sparse_mla_decode(pool, ids, q, 0.05)
    b = sm.sparse_mla_decode(pool, ids[:, rs.permutation(33)], q, 0.05)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def _brute(pool, ids, q_bits, scale):
    """Scalar loops: every byte decoded on its own, sums by hand."""
    T, H = q_bits.shape[:2]
    out = [[[0.0] * 512 for _ in range(H)] for _ in range(T)]
    lse = [[-math.inf] * H for _ in range(T)]
    for t in range(T):
        rows = [int(i) for i in ids[t] if 0 <= int(i) < pool.shape[0]]
        keys, vals = [], []
        for i in rows:
            r = pool[i]
            sc = [float(np.frombuffer(r[512 + 4 * j:516 + 4 * j].tobytes(), "<f4")[0])
                  for j in range(4)]
            lat = [sm.fp8_e4m3_value(int(r[d])) * sc[d // 128] for d in range(512)]
            rope = [float(sm.bf16_to_float(np.frombuffer(r[528 + 2 * d:530 + 2 * d].tobytes(),
                                                         "<u2"))[0]) for d in range(64)]
            keys.append(lat + rope)
            vals.append(lat)
        for h in range(H):
            if not rows:
                continue
            qh = [float(x) for x in sm.bf16_to_float(q_bits[t, h])]
            s = [scale * sum(a * b for a, b in zip(qh, k)) for k in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = sum(w)
            out[t][h] = [sum(w[j] * vals[j][d] for j in range(len(rows))) / z for d in range(512)]
            lse[t][h] = mx + math.log(z)
    return np.array(out), np.array(lse)


def test_matches_scalar_restatement():
    rs = np.random.default_rng(4)
    pool, q = _pool(rs, 9), _q(rs, 2, 2)
    ids = np.array([[3, 8, -1, 3, 0, 12], [5, 5, 2, 7, -3, 1]], np.int32)
    out, lse = sm.sparse_mla_decode(pool, ids, q, 0.07)
    bo, bl = _brute(pool, ids, q, 0.07)
    assert np.allclose(out, bo, rtol=1e-12, atol=1e-12) and np.allclose(lse, bl, rtol=1e-12)


# ---- planted mistakes (in copies of the oracle's steps, on the CPU) -------

def _mutant_decode_tiles_interleaved(rows):
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    table = np.array([sm.fp8_e4m3_value(b) for b in range(256)])
    sc = rows[:, 512:528].copy().view("<f4").astype(np.float64)
    lat = table[rows[:, :512]] * np.tile(sc, 128)            # scale t on every 4th value
    rope = sm.bf16_to_float(rows[:, 528:].copy().view("<u2"))
    return np.concatenate([lat, rope], axis=1), lat


_decode = sm.decode_rows


def _mutant_decode_no_rope(rows):
    k, v = _decode(rows)
    k = k.copy()
    k[:, 512:] = 0.0
    return k, v


@pytest.mark.parametrize("mutant", [_mutant_decode_tiles_interleaved, _mutant_decode_no_rope])
def test_pins_catch_planted_decode_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(sm, "decode_rows", mutant)
    failed = 0
    for pin in (test_decode_hand_built_row, test_matches_scalar_restatement):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


def _mutant_attention_dedups(pool, row_ids, q_bits, sm_scale):
    ids = np.array([np.r_[np.unique(r[r >= 0]), np.full((r < 0).sum(), -1)]
                    for r in row_ids.astype(np.int64)], dtype=np.int32)
    return _attend(pool, ids, q_bits, sm_scale)


def _mutant_attention_lse_unshifted(pool, row_ids, q_bits, sm_scale):
    out, lse = _attend(pool, row_ids, q_bits, sm_scale)
    return out, lse - np.nan_to_num(lse.max(axis=1, keepdims=True), neginf=0.0) * 0 - 0.5


_attend = sm.sparse_mla_decode


@pytest.mark.parametrize("mutant", [_mutant_attention_dedups, _mutant_attention_lse_unshifted])
def test_pins_catch_planted_attention_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(sm, "sparse_mla_decode", mutant)
    failed = 0
    for pin in (test_one_selected_row_is_its_value, test_equal_scores_average_and_duplicates_weigh_double,
                test_matches_scalar_restatement):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
