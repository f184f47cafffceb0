"""Pins of the oracle's bf16 rounding: a library routine and exact arithmetic."""
from fractions import Fraction

import numpy as np
import torch

from oracle.numerics import bf16_round, bf16_bits, from_bf16_bits


def nearest_bf16_exact(x: Fraction) -> Fraction:
    """Brute force: the nearest value with 8 significant bits, ties to even."""
    if x == 0:
        return Fraction(0)
    sign = 1 if x > 0 else -1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128                      # in [128, 256)
    lo = scaled.numerator // scaled.denominator
    frac = scaled - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Fraction(lo, 128) * Fraction(2) ** e


def test_matches_torch_bfloat16_on_fp32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(bf16_round(x.astype(np.float64)), want)


def test_ties_to_even_and_no_double_rounding():
    one = 1.0
    assert bf16_round(np.array([one + 2**-8]))[0] == 1.0                 # tie -> even
    assert bf16_round(np.array([one + 3 * 2**-8]))[0] == one + 2**-6     # tie -> even (up)
    # just above a tie in float64 but a tie after an fp32 rounding: must go up
    assert bf16_round(np.array([one + 2**-8 + 2**-40]))[0] == one + 2**-7


def test_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(2000) * 10
    got = bf16_round(xs)
    for x, g in zip(xs, got):
        assert Fraction(g) == nearest_bf16_exact(Fraction(float(x)))


def test_bits_roundtrip():
    v = bf16_round(np.array([1.5, -0.75, 3.140625]))
    assert list(bf16_bits(v)) == [0x3FC0, 0xBF40, 0x4049]
    assert np.array_equal(from_bf16_bits(bf16_bits(v)), v)
