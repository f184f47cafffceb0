"""Default selector and compact positions.

KVMem paper, Sec. 4.3: the configured sink and recent regions are always
kept; the rest of the budget goes to the blocks with the largest R_b; the
selection is then put back in chronological order. Sec. 4.4 and Sec. 5: the
selected blocks, in chronological order, get contiguous positions in the
compact execution window.

Readings: the budget counts blocks (token budget / block size); sink = the
first n_sink blocks, recent = the last n_recent blocks; k = budget - n_sink -
n_recent; exact ties go to the lower block index; when N <= budget every
block is kept; budget < n_sink + n_recent is an error; scores must be finite
and non-negative. Block i of the selection (0-based, ascending) occupies
positions B*i .. B*i + B - 1.
"""
from __future__ import annotations

import numpy as np


def select_blocks(R: np.ndarray, n_sink: int, n_recent: int, budget: int) -> np.ndarray:
    R = np.asarray(R)
    N = R.shape[0]
    if n_sink < 0 or n_recent < 0 or budget < 0:
        raise ValueError("negative size")
    if not np.all(np.isfinite(R)) or np.any(R < 0):
        raise ValueError("scores must be finite and non-negative")
    if n_sink + n_recent > budget:
        raise ValueError("budget smaller than sink + recent")
    if N <= budget:
        return np.arange(N, dtype=np.int64)
    forced = np.r_[np.arange(0, n_sink), np.arange(N - n_recent, N)]
    cand = np.arange(n_sink, N - n_recent)
    k = budget - n_sink - n_recent
    # order candidates by score descending; a stable sort keeps the lower
    # index first among exact ties
    order = np.argsort(-R[cand], kind="stable")
    chosen = cand[order[:k]]
    return np.sort(np.r_[forced, chosen]).astype(np.int64)


def compact_positions(n_sel: int, block_tokens: int = 32) -> np.ndarray:
    """First position of each selected block in the compact window."""
    return np.arange(n_sel, dtype=np.int64) * block_tokens


def cutoff_margin(R: np.ndarray, n_sink: int, n_recent: int, budget: int) -> float:
    """Relative gap (R_(k) - R_(k+1)) / R_(k) between the last selected and the
    first rejected candidate; inf when nothing is rejected."""
    R = np.asarray(R, dtype=np.float64)
    N = R.shape[0]
    if N <= budget:
        return float("inf")
    cand = R[n_sink:N - n_recent]
    k = budget - n_sink - n_recent
    if k <= 0 or k >= cand.shape[0]:
        return float("inf")
    s = np.sort(cand)[::-1]
    if s[k - 1] == 0:
        return 0.0
    return float((s[k - 1] - s[k]) / s[k - 1])
