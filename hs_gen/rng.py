"""Counter-based random numbers for the synthetic workloads.

Every random draw in the workloads is ``splitmix64`` (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
published by S. Vigna) applied to a 64-bit counter, keyed by a chain of
``splitmix64`` mixes of small integers (config seed, request, layer, step,
purpose).  Nothing here knows anything about KV caches: this module only turns
keys and counters into integers.

Three implementations of the same function are given -- Python ints for keys,
numpy ``uint64`` for vectors, torch ``int64`` (two's-complement wraparound) for
bulk content on any device -- and a CPU test checks that they agree.
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB


def splitmix64(x: int) -> int:
    """splitmix64 finaliser of (x + gamma), Python ints."""
    z = (x + GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def key(*parts: int) -> int:
    """Fold a sequence of small integers into one 64-bit key."""
    h = 0x243F6A8885A308D3  # arbitrary non-zero start value
    for p in parts:
        h = splitmix64(h ^ splitmix64(int(p) & MASK64))
    return h


def splitmix64_np(x: np.ndarray) -> np.ndarray:
    """Vectorised splitmix64 on uint64 arrays (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = x.astype(np.uint64, copy=True) + np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        return z ^ (z >> np.uint64(31))


def draws(k: int, start: int, count: int) -> np.ndarray:
    """``count`` uint64 draws of stream ``k``, counters start..start+count-1."""
    with np.errstate(over="ignore"):
        ctr = np.uint64(k) + np.arange(start, start + count, dtype=np.uint64)
    return splitmix64_np(ctr)


def _signed(c: int) -> int:
    return c - (1 << 64) if c >= (1 << 63) else c


def splitmix64_torch(x):
    """splitmix64 on torch int64 tensors; bit-identical to the uint64 form."""
    z = x + _signed(GAMMA)
    z = (z ^ ((z >> 30) & ((1 << 34) - 1))) * _signed(M1)
    z = (z ^ ((z >> 27) & ((1 << 37) - 1))) * _signed(M2)
    return z ^ ((z >> 31) & ((1 << 33) - 1))


def uniform_ints(k: int, start: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers in [lo, hi) (modulo reduction; bias < 2^-40 here)."""
    span = hi - lo
    if span <= 0:
        raise ValueError("empty range")
    return (draws(k, start, count) % np.uint64(span)).astype(np.int64) + lo


def permutation(k: int, n: int) -> np.ndarray:
    """A seeded permutation of range(n): argsort of n keyed draws."""
    return np.argsort(draws(k, 0, n), kind="stable").astype(np.int64)
