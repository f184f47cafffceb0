"""Pins of re-RoPE (KVMem paper Sec. 4.4; InferScale paper Sec. 2.4, Theorem 6)."""
import math

import numpy as np

from oracle import rope_frequencies, rope_rotate, rope_matrix


def test_identity_at_position_zero_and_norm_preserved():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 64))
    assert np.array_equal(rope_rotate(x, np.zeros(5)), x)
    y = rope_rotate(x, np.array([1, 77, 1000, 131071, 9999999]))
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_two_dims_is_the_plane_rotation():
    # d = 2: theta_0 = 1, so position p rotates by p radians
    for p in (1, 2, 5, 100):
        x, y = 0.3, -1.7
        got = rope_rotate(np.array([[x, y]]), np.array([p]))[0]
        want = [x * math.cos(p) - y * math.sin(p), x * math.sin(p) + y * math.cos(p)]
        assert np.allclose(got, want, rtol=1e-14, atol=1e-15)


def test_frequencies_closed_form():
    th = rope_frequencies(128)
    assert th[0] == 1.0
    assert math.isclose(th[1], math.pow(10000.0, -1 / 64), rel_tol=1e-15)
    assert math.isclose(th[63], math.pow(10000.0, -126 / 128), rel_tol=1e-15)


def test_complex_form_equals_block_diagonal_matrix_form():
    rng = np.random.default_rng(12)
    for layout in (0, 1):
        x = rng.standard_normal(32)
        for p in (3, 4097, 65535):
            got = rope_rotate(x[None], np.array([p]), layout=layout)[0]
            want = rope_matrix(p, 32, layout=layout) @ x
            assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_composition_and_relative_position_identity():
    rng = np.random.default_rng(13)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for a, b in [(0, 5), (17, 3), (123456, 9999999), (10_000_000, 1)]:
        ra = rope_rotate(rope_rotate(k[None], [a]), [b])
        assert np.allclose(ra, rope_rotate(k[None], [a + b]), rtol=0, atol=1e-9)
        lhs = float(rope_rotate(q[None], [a])[0] @ rope_rotate(k[None], [b])[0])
        rhs = float(q @ rope_rotate(k[None], [b - a])[0])
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_shift_equivalence_theorem6_item1():
    rng = np.random.default_rng(14)
    q, ks = rng.standard_normal(64), rng.standard_normal((32, 64))
    N, v0, p0 = 5000, 1200, 870000
    Np = N - (v0 - p0)
    j = np.arange(32)
    lhs = rope_rotate(ks, v0 + j) @ rope_rotate(q[None], [N])[0]
    rhs = rope_rotate(ks, p0 + j) @ rope_rotate(q[None], [Np])[0]
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)


def test_layouts_differ_by_a_fixed_permutation():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 16))
    perm = np.r_[np.arange(0, 16, 2), np.arange(1, 16, 2)]  # interleaved -> half-split
    pos = np.array([1, 9, 300, 4000])
    a = rope_rotate(x, pos, layout=0)[:, perm]
    b = rope_rotate(x[:, perm], pos, layout=1)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


# ---- bounded delta re-RoPE (KVMem Sec. 4.4) ----

def _bf16_block(seed, shape=(2, 32, 16)):
    from oracle.numerics import bf16_round
    return bf16_round(np.random.default_rng(seed).standard_normal(shape))


def _ulp_bf16(x):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -100))) - 7)


def test_delta_limit_zero_is_reencoding_from_raw_every_time():
    from oracle import bounded_delta_rope
    from oracle.numerics import bf16_round
    k = _bf16_block(21)
    P = [64, 96, 0, 320, 320, 32]
    xs, kinds, counts = bounded_delta_rope(k, P, 0, "bf16")
    assert kinds == ["full", "full", "full", "full", "same", "full"]
    assert counts == [0] * 6
    for x, p in zip(xs, P):
        assert np.array_equal(x, bf16_round(rope_rotate(k, p + np.arange(32))))


def test_delta_steps_compose_exactly_without_rounding():
    """R_a R_b = R_{a+b}: unrounded delta steps land on the direct rotation."""
    from oracle import bounded_delta_rope
    k = np.random.default_rng(22).standard_normal((2, 32, 16))
    P = [0, 4096, 33, 100000, 7]
    for layout in (0, 1):
        xs, kinds, _ = bounded_delta_rope(k, P, 10, "f64", layout=layout)
        assert kinds == ["full"] + ["delta"] * 4
        for x, p in zip(xs, P):
            assert np.max(np.abs(x - rope_rotate(k, p + np.arange(32), layout=layout))) <= 1e-11


def test_counter_resets_after_the_limit():
    from oracle import bounded_delta_rope
    from oracle.numerics import bf16_round
    k = _bf16_block(23)
    P = [0, 32, 64, 96, 128, 160, 160, 192, 224]
    xs, kinds, counts = bounded_delta_rope(k, P, 2, "bf16")
    assert kinds == ["full", "delta", "delta", "full", "delta", "delta", "same", "full", "delta"]
    assert counts == [0, 1, 2, 0, 1, 2, 2, 0, 1]
    for x, p, kind in zip(xs, P, kinds):
        if kind == "full":
            assert np.array_equal(x, bf16_round(rope_rotate(k, p + np.arange(32))))


def test_delta_error_grows_at_most_half_ulp_per_pair_per_store():
    """Each store rounds both components of a pair by at most half an ulp, and
    a rotation keeps earlier error's length, so after n deltas the pair error
    is at most (n + 1) * sqrt(2)/2 ulp of the pair's length (bf16)."""
    from oracle import bounded_delta_rope
    k = _bf16_block(24, (4, 32, 64))
    P = [0, 3000, 17, 9000, 450, 120000, 64, 5000, 99]
    for layout in (0, 1):
        xs, _, counts = bounded_delta_rope(k, P, 8, "bf16", layout=layout)
        worst = []
        for n, (x, p) in enumerate(zip(xs, P)):
            exact = rope_rotate(k, p + np.arange(32), layout=layout)
            if layout == 0:
                ea, eb, na, nb = (x - exact)[..., 0::2], (x - exact)[..., 1::2], exact[..., 0::2], exact[..., 1::2]
            else:
                ea, eb, na, nb = (x - exact)[..., :32], (x - exact)[..., 32:], exact[..., :32], exact[..., 32:]
            err = np.hypot(ea, eb)
            norm = np.hypot(na, nb)
            bound = (counts[n] + 1) * (np.sqrt(2) / 2) * _ulp_bf16(1.1 * norm)
            assert np.all(err <= bound)
            worst.append(float(np.max(err / _ulp_bf16(norm))))
        assert worst[-1] > worst[0]          # the error does grow with the deltas
