"""Pins of Mean-K (KVMem paper Sec. 4.3; incremental indexing Sec. 5)."""
import math
from fractions import Fraction

import numpy as np

import synth
from oracle import mean_k, mean_k_index
from oracle.numerics import bf16_round
from oracle.pipeline import index_rows, raw_blocks
from tests.test_oracle_numerics import nearest_bf16_exact


def test_each_entry_is_the_exactly_rounded_block_mean():
    rng = np.random.default_rng(2)
    k = bf16_round(rng.standard_normal((2, 2, 3, 32, 8)))        # [nb][L][Hkv][B][d]
    idx = mean_k_index(k, "bf16")                                 # [L][Hkv][nb][d]
    for b in range(2):
        for l in range(2):
            for g in range(3):
                for t in range(8):
                    exact = sum(Fraction(float(k[b, l, g, j, t])) for j in range(32)) / 32
                    assert Fraction(float(idx[l, g, b, t])) == nearest_bf16_exact(exact)


def test_closed_form_symmetric_block():
    v = np.array([0.5, -2.0, 3.25, 0.0])
    c = np.array([0.125, 0.25, -0.5, 1.0])
    k = np.stack([v + (j - 15.5) * c for j in range(32)])[None, None, None]   # mean is v
    assert np.array_equal(mean_k(k, "f32")[0, 0, 0], v)


def test_linearity_q_dot_mean_equals_mean_of_q_dot_k():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, 1, 32, 64)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal(64)
    kbar = k.sum(axis=3) / 32                     # what mean_k rounds
    stored = mean_k(k, "f32")[0, 0, 0]
    lhs = float(q @ stored)
    rhs = math.fsum(float(q @ k[0, 0, 0, j]) for j in range(32)) / 32
    bound = float(np.abs(q) @ np.abs(stored - kbar[0, 0, 0])) + 1e-12
    assert abs(lhs - rhs) <= bound
    assert np.max(np.abs(stored - kbar[0, 0, 0])) <= 2**-24 * np.max(np.abs(kbar)) * 2


def test_incremental_append_equals_full_build():
    wl = synth.get_workload("ctx64k").scaled(n_layers=2)
    full = index_rows(wl, 0, 40, chunk=16)
    a = index_rows(wl, 0, 25, chunk=16)
    b = index_rows(wl, 25, 15, chunk=16)
    assert np.array_equal(full, np.concatenate([a, b], axis=2))


def test_layout_is_layer_head_block_dim():
    wl = synth.get_workload("tiny")
    idx = index_rows(wl, 0, 4)
    k = raw_blocks(wl, "K", 2, 1)[0]              # [L][Hkv][B][d]
    for g in range(2):
        want = np.array([math.fsum(k[0, g, :, t]) / 32 for t in range(64)])
        assert np.array_equal(idx[0, g, 2], want.astype(np.float32).astype(np.float64))


# ---- Mean-K from K that already carries RoPE (KVMem Sec. 5) ----

def _rope_blocks(k_raw, pos0, layout, base=10000.0):
    """Rotate block-major raw K [nb][L][Hkv][B][d] to its original positions."""
    from oracle import rope_rotate
    B = k_raw.shape[3]
    return np.stack([rope_rotate(k_raw[i], pos0 + B * i + np.arange(B), base, layout)
                     for i in range(k_raw.shape[0])])


def test_derope_mean_inverts_rope_exactly():
    from oracle import mean_k_from_rope
    rng = np.random.default_rng(11)
    k_raw = rng.standard_normal((3, 1, 2, 32, 16))
    for layout in (0, 1):
        for pos0 in (0, 1000, 9_999_968):
            k_rope = _rope_blocks(k_raw, pos0, layout)
            got = mean_k_from_rope(k_rope, pos0, "f64", layout=layout, table_fp32=False)
            want = k_raw.mean(axis=3)
            assert np.max(np.abs(got - want)) <= 1e-12


def test_derope_mean_equals_explicit_inverse_matrices():
    from oracle import mean_k_from_rope, rope_matrix
    rng = np.random.default_rng(12)
    k = rng.standard_normal((2, 1, 1, 32, 8))
    for layout in (0, 1):
        got = mean_k_from_rope(k, 77, "f64", layout=layout, table_fp32=False)
        for i in range(2):
            acc = np.zeros(8)
            for j in range(32):
                acc += rope_matrix(77 + 32 * i + j, 8, layout=layout).T @ k[i, 0, 0, j]
            assert np.max(np.abs(got[i, 0, 0] - acc / 32)) <= 1e-13


def test_derope_unit_vectors_hand_case():
    """d = 2: theta_0 = 1, so token j at position p_j = (cos p_j, sin p_j) turns
    back into (1, 0) and the block mean is (1, 0)."""
    from oracle import mean_k_from_rope
    p = 5 + np.arange(32)
    k = np.stack([np.cos(p), np.sin(p)], axis=-1)[None, None, None]     # [1][1][1][32][2]
    got = mean_k_from_rope(k, 5, "f64", table_fp32=False)[0, 0, 0]
    assert np.max(np.abs(got - [1.0, 0.0])) <= 1e-15
    # with the fp32 table the second component is the table's rounding residue
    tab = mean_k_from_rope(k, 5, "bf16")[0, 0, 0]
    assert tab[0] == 1.0 and abs(tab[1]) <= 2.0 ** -24


def test_derope_fp32_table_error_bound():
    """Rounding cos/sin to fp32 moves each de-rotated value by at most
    (|a| + |b|) * 2^-25 (half an fp32 ulp of a value below 1, twice)."""
    from oracle import mean_k_from_rope
    rng = np.random.default_rng(13)
    k = rng.standard_normal((2, 2, 2, 32, 16))
    for layout in (0, 1):
        exact = mean_k_from_rope(k, 123456, "f64", layout=layout, table_fp32=False)
        table = mean_k_from_rope(k, 123456, "f64", layout=layout, table_fp32=True)
        a = k[..., 0::2] if layout == 0 else k[..., :8]
        b = k[..., 1::2] if layout == 0 else k[..., 8:]
        bound = ((np.abs(a) + np.abs(b)).mean(axis=3)).max() * 2.0 ** -24
        assert 0 < np.max(np.abs(exact - table)) <= bound
