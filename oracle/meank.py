"""Mean-K block representation.

KVMem paper, Sec. 4.3 ("what to recall"): for every layer l and KV head g, a
historical block b is represented by the mean of the position-independent
(pre-RoPE) K vectors of its tokens. The displayed formula was lost; the
reading is the unweighted arithmetic mean over the block's B tokens. Only
complete blocks are indexed (Sec. 5, incremental indexing of completed
blocks). The stored index has the K dtype; the mean is formed in float64 and
rounded once (round-to-nearest-even) into that dtype.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to_dtype
from .rope import rope_frequencies


def mean_k(k_raw_blocks: np.ndarray, dtype: str) -> np.ndarray:
    """k_raw_blocks: [nb][L][Hkv][B][d] float64 values of the stored raw K.

    Returns [nb][L][Hkv][d] float64 holding the stored (rounded) Mean-K."""
    k = np.asarray(k_raw_blocks, dtype=np.float64)
    m = k.sum(axis=3) / k.shape[3]
    return round_to_dtype(m, dtype)


def mean_k_index(k_raw_blocks: np.ndarray, dtype: str) -> np.ndarray:
    """The same Mean-K laid out as the scoring index [L][Hkv][nb][d]."""
    return np.ascontiguousarray(np.transpose(mean_k(k_raw_blocks, dtype), (1, 2, 0, 3)))


def mean_k_from_rope(k_rope_blocks: np.ndarray, pos0: int, dtype: str, base: float = 10000.0,
                     layout: int = 0, table_fp32: bool = True) -> np.ndarray:
    """Mean-K of blocks whose stored K already carries RoPE.

    KVMem Sec. 5: during prefill the engine removes RoPE from the K of completed
    blocks and forms their Mean-K while that K is still on the GPU. Block i of
    k_rope_blocks [nb][L][Hkv][B][d] holds tokens at original positions
    pos0 + B*i + j. Each token is rotated back by R_{-p} (the inverse of the
    rotation in ``oracle.rope``), then the block mean is taken in float64 and
    rounded once into the index dtype.

    Reading: cos and sin of the float64 angle p * theta_t are rounded to fp32
    (the precision of the table that also drives re-RoPE) when table_fp32 is
    set; the de-rotation itself is float64. table_fp32=False uses the float64
    values, which makes R_{-p} the exact inverse of ``rope_rotate``."""
    k = np.asarray(k_rope_blocks, dtype=np.float64)
    nb, B, d = k.shape[0], k.shape[3], k.shape[4]
    pos = pos0 + B * np.arange(nb)[:, None] + np.arange(B)[None, :]          # [nb][B]
    ang = pos[..., None].astype(np.float64) * rope_frequencies(d, base)      # [nb][B][d/2]
    c, s = np.cos(ang), np.sin(ang)
    if table_fp32:
        c, s = c.astype(np.float32).astype(np.float64), s.astype(np.float32).astype(np.float64)
    c = c[:, None, None, :, :]
    s = s[:, None, None, :, :]
    if layout == 0:
        a, b = k[..., 0::2], k[..., 1::2]
    else:
        a, b = k[..., : d // 2], k[..., d // 2:]
    a0 = a * c + b * s          # R_{-p}: rotate each (a, b) pair by -p * theta_t
    b0 = b * c - a * s
    out = np.empty_like(k)
    if layout == 0:
        out[..., 0::2], out[..., 1::2] = a0, b0
    else:
        out[..., : d // 2], out[..., d // 2:] = a0, b0
    return round_to_dtype(out.sum(axis=3) / B, dtype)
