"""Re-application of rotary position embedding (RoPE) to raw K.

KVMem paper, Sec. 4.4: an incoming block gets RoPE applied to its immutable
raw (position-independent) K at its newly assigned compact position; V is
copied unchanged. The rotation itself follows the InferScale paper, Sec. 2.4
and Theorem 6: a fixed block-diagonal rotation R_p built from 2x2 rotations
by angles p * theta_t.

Readings: theta_t = base ** (-2t/d), t = 0 .. d/2-1, base 10000 (RoFormer
form); the 2x2 blocks pair dims (2t, 2t+1) ("interleaved", layout 0) or
(t, t + d/2) ("half-split", layout 1). The rotated value is kept in float64,
unrounded.
"""
from __future__ import annotations

import numpy as np


def rope_frequencies(d: int, base: float = 10000.0) -> np.ndarray:
    t = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * t / d)


def _pairs(x: np.ndarray, layout: int):
    d = x.shape[-1]
    if layout == 0:
        return x[..., 0::2], x[..., 1::2]
    return x[..., : d // 2], x[..., d // 2:]


def _unpairs(a: np.ndarray, b: np.ndarray, layout: int) -> np.ndarray:
    out = np.empty(a.shape[:-1] + (2 * a.shape[-1],), dtype=np.float64)
    if layout == 0:
        out[..., 0::2] = a
        out[..., 1::2] = b
    else:
        h = a.shape[-1]
        out[..., :h] = a
        out[..., h:] = b
    return out


def rope_rotate(x: np.ndarray, pos, base: float = 10000.0, layout: int = 0) -> np.ndarray:
    """Rotate vectors x[..., P, d] at positions pos[P] (complex form).

    Each pair (a, b) is read as a + i*b and multiplied by exp(i * p * theta_t)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[:, None] * rope_frequencies(d, base)[None, :]        # [P][d/2]
    a, b = _pairs(x, layout)
    z = (a + 1j * b) * np.exp(1j * ang)
    return _unpairs(z.real, z.imag, layout)


def rope_matrix(p: float, d: int, base: float = 10000.0, layout: int = 0) -> np.ndarray:
    """The d x d rotation R_p as an explicit matrix (block-diagonal form)."""
    th = rope_frequencies(d, base)
    M = np.zeros((d, d))
    for t in range(d // 2):
        i, j = (2 * t, 2 * t + 1) if layout == 0 else (t, t + d // 2)
        c, s = np.cos(p * th[t]), np.sin(p * th[t])
        M[i, i], M[i, j], M[j, i], M[j, j] = c, -s, s, c
    return M


def bounded_delta_rope(k_raw: np.ndarray, base_positions, limit: int, dtype: str,
                       base: float = 10000.0, layout: int = 0):
    """Stored K of one block over a sequence of compact placements, with
    bounded delta re-RoPE (KVMem Sec. 4.4).

    k_raw [..., B, d]: the block's raw (pre-RoPE) K; token j of placement i sits
    at base_positions[i] + j. Placement 0 encodes from raw K. Later, when the
    position changes, the stored low-precision K is rotated in place by the
    shift delta = P_i - P_{i-1} (the same for every token) and rounded again,
    at most `limit` times in a row; the change after that reconstructs from raw
    K at the new position and resets the counter. An unchanged position leaves
    K (and the counter) as it is. Rotations are float64, each store is one
    round-to-nearest-even into dtype ("f64": no rounding).

    Returns (stored K per placement, kind per placement: "full", "delta" or
    "same", delta count after each placement)."""
    k = np.asarray(k_raw, dtype=np.float64)
    B = k.shape[-2]
    j = np.arange(B)
    out, kinds, counts = [], [], []
    x, prev, n = None, None, 0
    for i, p in enumerate(base_positions):
        if i == 0 or (p != prev and n >= limit):
            x = round_store(rope_rotate(k, p + j, base, layout), dtype)
            kind, n = "full", 0
        elif p == prev:
            kind = "same"
        else:
            x = round_store(rope_rotate(x, np.full(B, p - prev), base, layout), dtype)
            kind, n = "delta", n + 1
        out.append(x)
        kinds.append(kind)
        counts.append(n)
        prev = p
    return out, kinds, counts


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    from .numerics import round_to_dtype
    return round_to_dtype(x, dtype)
