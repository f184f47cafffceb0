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


# ---- FP8 E4M3FN ----

def test_fp8_decode_table_landmarks():
    from oracle.numerics import fp8_decode
    v = fp8_decode(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0           # largest finite
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9    # smallest normal / subnormal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x40] == 2.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])          # the only NaNs, no infinities
    fin = v[:0x7F]
    assert np.all(np.diff(fin) > 0)                          # codes 0..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -fin[:0x7F])


def test_fp8_encode_exact_nearest_ties_even_saturate():
    from fractions import Fraction
    from oracle.numerics import fp8_decode, fp8_encode
    vals = [Fraction(float(x)) for x in fp8_decode(np.arange(0x7F, dtype=np.uint8))]
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(400) * 3, rng.standard_normal(200) * 0.01,
                         (np.array(vals[1:], dtype=float) + np.array(vals[:-1], dtype=float)) / 2])
    for x in xs:
        a = min(Fraction(abs(float(x))), Fraction(448))
        d = [abs(a - v) for v in vals]
        best = min(range(len(vals)), key=lambda i: (d[i], i % 2))   # nearest, even code on ties
        code = int(fp8_encode(x))
        assert code & 0x7F == best and (code >> 7) == (1 if np.signbit(x) else 0)
    assert fp8_encode(1000.0) == 0x7E and fp8_encode(-1e9) == 0xFE
    assert fp8_encode(-0.0) == 0x80 and fp8_encode(-1e-6) == 0x80


def test_fp8_round_trip_of_every_finite_code():
    from oracle.numerics import fp8_decode, fp8_encode
    fin = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8_encode(fp8_decode(fin)), fin)


def test_round_to_fp8_is_nearest_e4m3_value():
    """Page stores in FP8 (the bounded delta re-RoPE model of FP8 pages) round
    to the nearest E4M3 value, ties to the even code, saturating at 448."""
    from oracle.numerics import round_to_dtype
    x = np.array([1.0625, 1.1, 1.1875, -3.3, 500.0, -1e9, 2.0 ** -10, 3 * 2.0 ** -10,
                  0.0, 2.0 ** -9, 240.0, 0.013])
    want = np.array([1.0, 1.125, 1.25, -3.25, 448.0, -448.0, 0.0, 2.0 ** -8,
                     0.0, 2.0 ** -9, 240.0, 0.013671875])
    got = round_to_dtype(x, "fp8")
    assert np.array_equal(got, want)
    assert np.array_equal(round_to_dtype(got, "fp8"), got)
