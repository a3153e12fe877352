"""Synthetic KV row content.

A KV row is 656 opaque bytes (an assumed sparse-MLA layout: 512 B of fp8
latent, 16 B of scales, 128 B of rope; nothing on the hot path looks inside).
The synthetic row of token ``t`` of source sequence ``src`` in layer ``l`` is
82 little-endian 64-bit words ``splitmix64(h + k)``, k = 0..81, where ``h`` is a
splitmix64 chain over (seed, l, src, t).  Because every row can be recomputed
from its (l, src, t) alone, a gathered row can be checked against what its
token must hold without reference to any resolver.
"""

from __future__ import annotations

import numpy as np
import torch

from .rng import splitmix64_np, splitmix64_torch

ROW_BYTES = 656
ROW_WORDS = ROW_BYTES // 8
PAGE = 64
CONTENT_SEED = 0x5EED_C0DE


def _head_np(layer, src, tok):
    h = splitmix64_np(np.asarray(tok, dtype=np.int64).astype(np.uint64))
    h = splitmix64_np(np.asarray(src, dtype=np.int64).astype(np.uint64) ^ h)
    h = splitmix64_np(np.asarray(layer, dtype=np.int64).astype(np.uint64) ^ h)
    return splitmix64_np(np.uint64(CONTENT_SEED) ^ h)


def content_np(layer, src, tok) -> np.ndarray:
    """uint8 [n, 656] rows for broadcastable (layer, src, tok) arrays (numpy)."""
    layer, src, tok = np.broadcast_arrays(np.atleast_1d(layer), np.atleast_1d(src),
                                          np.atleast_1d(tok))
    h = _head_np(layer.ravel(), src.ravel(), tok.ravel())
    with np.errstate(over="ignore"):
        w = splitmix64_np(h[:, None] + np.arange(ROW_WORDS, dtype=np.uint64)[None, :])
    return w.astype("<u8").view(np.uint8).reshape(-1, ROW_BYTES)


def content_torch(layer, src, tok) -> torch.Tensor:
    """Same rows as :func:`content_np` from int64 tensors on any device."""
    dev = tok.device
    h = splitmix64_torch(tok.to(torch.int64))
    h = splitmix64_torch(src.to(torch.int64) ^ h)
    h = splitmix64_torch(layer.to(torch.int64) ^ h)
    h = splitmix64_torch(torch.full_like(h, CONTENT_SEED) ^ h)
    k = torch.arange(ROW_WORDS, dtype=torch.int64, device=dev)
    w = splitmix64_torch(h[:, None] + k[None, :])
    return w.contiguous().view(torch.uint8).reshape(-1, ROW_BYTES)


def fill_rows(dst: torch.Tensor, rows: torch.Tensor, layer: int, src: torch.Tensor,
              tok: torch.Tensor, chunk: int = 1 << 16, compute_device=None) -> None:
    """Write content(layer, src[i], tok[i]) into row ``rows[i]`` of ``dst``.

    ``dst`` is a uint8 [n_rows, 656] view of one layer of a pool (any device);
    ``rows``, ``src`` and ``tok`` are int64 tensors of equal length.  The
    content is computed on ``compute_device`` (default: dst's device) and
    copied into ``dst``.
    """
    n = rows.numel()
    dev = torch.device(compute_device) if compute_device is not None else dst.device
    if dev.type != "cpu" or dst.device.type != "cpu":
        chunk = max(chunk, 1 << 20)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        lay = torch.full((e - s,), layer, dtype=torch.int64, device=dev)
        rowsv = content_torch(lay, src[s:e].to(dev), tok[s:e].to(dev))
        dst.index_copy_(0, rows[s:e].to(dst.device), rowsv.to(dst.device))
