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
