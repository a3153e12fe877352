"""CPU oracle for sparse MLA decode over resolved rows read in place.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  Plain numpy in
float64; it shares nothing with the HIP library.

What it computes ("vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1"):
  * "Use sparsity when needed": hot pages live in the same KV-cache tensor as
    resident pages, so the sparse MLA kernel sees them as ordinary pages;
  * "How it works": the resolver hands back one HMA row id per selected
    token whether the row is resident or hot, and the kernel reads the rows
    at one stride -- here straight from the pool by row id, no gathered copy.

Readings (the pages fix neither the row format nor the attention numerics):
  * a row is 656 bytes of an FP8 MLA cache: 512 latent values as OCP FP8
    E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
    0x7F/0xFF NaN, no infinities), then 4 little-endian float32 scales, scale
    t applying to latent values [128 t, 128 t + 128), then 64 rope values as
    bfloat16;
  * a row's key is its 512 scaled latent values followed by its 64 rope
    values (576); its value is the 512 scaled latent values;
  * a query token has H heads of 576 bfloat16 values; for each head,
    s_j = sm_scale * <q, k_j> over the token's selected rows, out =
    sum_j softmax(s)_j v_j and lse = log(sum_j exp(s_j)) (natural log);
  * a row id outside [0, pool_rows) (padding -1, overflow -2, invalid -3)
    selects nothing; a token with no selected row gets out = 0, lse = -inf;
  * a row id listed twice counts twice.
"""

from __future__ import annotations

import numpy as np

ROW_BYTES = 656
LATENT = 512
ROPE = 64
TILE = 128
SCALE_OFF = 512
ROPE_OFF = 528


def fp8_e4m3_value(byte: int) -> float:
    """The value of one OCP FP8 E4M3 byte, from its fields."""
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9          # subnormal: m / 8 * 2^(1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_rows(rows: np.ndarray):
    """uint8 [n, 656] -> (keys float64 [n, 576], values float64 [n, 512])."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    table = np.array([fp8_e4m3_value(b) for b in range(256)], dtype=np.float64)
    lat = table[rows[:, :LATENT]]
    scales = rows[:, SCALE_OFF:SCALE_OFF + 16].copy().view("<f4").astype(np.float64)
    lat = lat * np.repeat(scales, TILE, axis=1)
    rope = bf16_to_float(rows[:, ROPE_OFF:ROW_BYTES].copy().view("<u2"))
    return np.concatenate([lat, rope], axis=1), lat


def sparse_mla_decode(pool: np.ndarray, row_ids: np.ndarray, q_bits: np.ndarray,
                      sm_scale: float):
    """pool uint8 [pool_rows, 656] (one layer); row_ids int32 [T, K];
    q_bits uint16 [T, H, 576] (bfloat16) -> (out float64 [T, H, 512],
    lse float64 [T, H])."""
    T, K = row_ids.shape
    H = q_bits.shape[1]
    out = np.zeros((T, H, LATENT), dtype=np.float64)
    lse = np.full((T, H), -np.inf, dtype=np.float64)
    for t in range(T):
        ids = row_ids[t].astype(np.int64)
        ids = ids[(ids >= 0) & (ids < pool.shape[0])]
        if ids.size == 0:
            continue
        k, v = decode_rows(pool[ids])
        q = bf16_to_float(q_bits[t])                       # [H, 576]
        s = sm_scale * (q @ k.T)                           # [H, n]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        z = w.sum(axis=1, keepdims=True)
        out[t] = (w / z) @ v
        lse[t] = (m + np.log(z))[:, 0]
    return out, lse
