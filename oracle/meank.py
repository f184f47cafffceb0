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


def mean_k(k_raw_blocks: np.ndarray, dtype: str) -> np.ndarray:
    """k_raw_blocks: [nb][L][Hkv][B][d] float64 values of the stored raw K.

    Returns [nb][L][Hkv][d] float64 holding the stored (rounded) Mean-K."""
    k = np.asarray(k_raw_blocks, dtype=np.float64)
    m = k.sum(axis=3) / k.shape[3]
    return round_to_dtype(m, dtype)


def mean_k_index(k_raw_blocks: np.ndarray, dtype: str) -> np.ndarray:
    """The same Mean-K laid out as the scoring index [L][Hkv][nb][d]."""
    return np.ascontiguousarray(np.transpose(mean_k(k_raw_blocks, dtype), (1, 2, 0, 3)))
