"""Storage rounding used by the oracle (its own definition; float64 in, exact out)."""
from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float64 values directly to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits. With x = m * 2**e and 0.5 <= |m| < 1,
    the rounded value is rint(m * 2**8) * 2**(e-8) (np.rint rounds half to
    even). Returned as float64 holding exactly representable bf16 values.
    Values below the bf16 normal range are not expected here and rejected."""
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    if nz.size and np.min(np.abs(nz)) < 2.0 ** -126:
        raise ValueError("bf16_round: subnormal input")
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_bits(x) -> np.ndarray:
    """Bit pattern (uint16) of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Store float64 values in the index dtype: bf16 (RNE) or fp32 (RNE); "f64"
    keeps the float64 value (used by pins that check identities exactly)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)
