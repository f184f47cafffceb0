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
    """Store float64 values in the index or page dtype: bf16 (RNE), fp32 (RNE)
    or fp8 (E4M3, nearest, ties to even, saturating; the page format of FP8 KV);
    "f64" keeps the float64 value (used by pins that check identities exactly)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "fp8":
        return fp8_decode(fp8_encode(x))
    raise ValueError(dtype)


# ---- FP8 E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
# no infinities, S.1111.111 is NaN, largest finite 448, subnormals m * 2^-9.

def fp8_decode(bits) -> np.ndarray:
    """Values of E4M3FN bytes (float64; NaN for 0x7F / 0xFF)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return s * val


def fp8_encode(x) -> np.ndarray:
    """Nearest E4M3FN byte, ties to even, saturating to +-448 (the largest
    finite value) beyond the range. Works on the exact float64 input: the
    finite codes are enumerated and the nearest one chosen, the even mantissa
    (lower code) on ties."""
    x = np.asarray(x, dtype=np.float64)
    codes = np.arange(0x7F, dtype=np.uint8)                 # 0 .. 448, ascending values
    vals = fp8_decode(codes)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(vals, a, side="left")             # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    exact = vals[hi] == a
    c = np.where(exact | pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(x), c | 0x80, c).astype(np.uint8)   # sign kept, also on zero


def fp8_round(x) -> np.ndarray:
    """x rounded to the nearest E4M3FN value (ties to even, saturating)."""
    return fp8_decode(fp8_encode(x))
