"""The generator of gen.c restated in plain NumPy (slow; for pinning only)."""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
UNIT_SCALE = np.uint32(0x37DDB3D7).view(np.float32)
INV_SQRT32 = np.uint32(0x3E3504F3).view(np.float32)


def mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def key(seed: int, tensor: int, i0: int, i1: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = mix64(np.uint64(seed) * GOLDEN + np.uint64(1))
        k = mix64(k + np.uint64(tensor + 1) * GOLDEN)
        k = mix64(k + np.uint64(i0 + 1) * GOLDEN)
        return mix64(k + np.uint64(i1 + 1) * GOLDEN)


def unit(k, e0: int, n: int) -> np.ndarray:
    e = np.arange(e0, e0 + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        h = mix64(np.uint64(k) + (e + np.uint64(1)) * GOLDEN)
    m = np.uint64(0xFFFF)
    s = ((h & m) + ((h >> np.uint64(16)) & m) + ((h >> np.uint64(32)) & m)
         + (h >> np.uint64(48))).astype(np.int64)
    return (s - 131070).astype(np.float32) * UNIT_SCALE


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
            ).astype(np.uint16)


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (OCP E4M3FN) codes of fp32 values: nearest, ties to even,
    saturating to +-448, sign kept."""
    x = np.asarray(x, dtype=np.float32)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x).astype(np.float32)
    sub = np.rint(a * np.float32(512.0)).astype(np.int64)            # below 2^-6
    f, e = np.frexp(a)                                                # a = f * 2^e
    E = e.astype(np.int64) - 1
    q = np.rint(np.ldexp(a, (3 - E).astype(np.int32))).astype(np.int64)
    E = np.where(q == 16, E + 1, E)
    q = np.where(q == 16, 8, q)
    norm = ((E + 7) << 3) | (q - 8)
    code = np.where(a < np.float32(0.015625), sub, norm)
    code = np.where((a >= np.float32(464.0)) | (E > 8) | ((E == 8) & (q > 14)), 0x7E, code)
    return (sign | code).astype(np.uint8)


def kv_block(seed, tensor, off_tensor, off_sigma, b, L, Hkv, B, d, dtype):
    out = np.empty((L, Hkv, B, d), dtype=np.float32)
    for l in range(L):
        for g in range(Hkv):
            lg = l * Hkv + g
            x = unit(key(seed, tensor, b, lg), 0, B * d).reshape(B, d)
            if off_sigma != 0.0:
                o = np.float32(off_sigma) * unit(key(seed, off_tensor, b, lg), 0, d)
                x = (x + o[None, :]).astype(np.float32)
            out[l, g] = x
    if dtype == "fp8":
        return to_e4m3_bits(out)
    return out if dtype == "f32" else to_bf16_bits(out)
