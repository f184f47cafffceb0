"""Pins of block relevance (KVMem paper Sec. 4.3, Eq. (10) as read from its prose)."""
import math

import numpy as np
import scipy.special

import synth
from oracle import block_scores, lg_partial_scores
from oracle.pipeline import run_step


def rand_case(rng, L=2, Hkv=2, G=3, T=4, N=37, d=16):
    q = rng.standard_normal((L, Hkv * G, T, d))
    idx = rng.standard_normal((L, Hkv, N, d))
    return q, idx


def test_scores_sum_to_number_of_query_tokens():
    rng = np.random.default_rng(4)
    for T in (1, 3, 7):
        q, idx = rand_case(rng, T=T)
        assert abs(block_scores(q, idx, threads=1).sum() - T) < 1e-12


def test_constant_index_gives_uniform_scores():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 3, 8))
    idx = np.broadcast_to(rng.standard_normal((2, 2, 1, 8)), (2, 2, 50, 8)).copy()
    assert np.allclose(block_scores(q, idx, threads=1), 3 / 50, rtol=0, atol=1e-15)


def test_single_row_is_the_textbook_softmax():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 1, 32))
    idx = rng.standard_normal((1, 1, 200, 32)) * 3
    want = scipy.special.softmax(idx[0, 0] @ q[0, 0, 0] / math.sqrt(32))
    assert np.allclose(block_scores(q, idx, threads=1), want, rtol=1e-13, atol=0)


def test_two_level_closed_form_pins_scale_group_map_and_average():
    # d = 4 (sqrt(d) = 2), L = 2, Hkv = 2, Hq = 4 (G = 2), T = 1, N = 3.
    # KV head g has one non-zero Mean-K: block b = g, equal to a*e0.
    # Query head h is c_h*e0, so its only non-zero score is c_h*a/2 on block g(h).
    L, Hkv, Hq, N, d, a = 2, 2, 4, 3, 4, 1.5
    c = {0: 1.0, 1: -2.0, 2: 0.5, 3: 3.0}
    idx = np.zeros((L, Hkv, N, d))
    q = np.zeros((L, Hq, 1, d))
    for l in range(L):
        for g in range(Hkv):
            idx[l, g, g, 0] = a
        for h in range(Hq):
            q[l, h, 0, 0] = c[h] * (l + 1)
    want = np.zeros(N)
    for l in range(L):
        for h in range(Hq):
            g = h // 2                               # grouped-query map
            x = c[h] * (l + 1) * a / 2.0
            z = math.exp(x) + (N - 1)
            for b in range(N):
                want[b] += (math.exp(x) if b == g else 1.0) / z
    want /= L * Hq
    assert np.allclose(block_scores(q, idx, threads=1), want, rtol=1e-14, atol=0)


def test_block_permutation_permutes_scores():
    rng = np.random.default_rng(7)
    q, idx = rand_case(rng)
    perm = rng.permutation(idx.shape[2])
    assert np.allclose(block_scores(q, idx[:, :, perm], threads=1),
                       block_scores(q, idx, threads=1)[perm], rtol=1e-13, atol=0)


def test_repeated_query_token_scales_scores():
    rng = np.random.default_rng(8)
    q, idx = rand_case(rng, T=1)
    q3 = np.repeat(q, 3, axis=2)
    assert np.allclose(block_scores(q3, idx, threads=1), 3 * block_scores(q, idx, threads=1),
                       rtol=1e-13, atol=0)


def test_partials_sum_to_group_rows_and_to_scores():
    rng = np.random.default_rng(9)
    q, idx = rand_case(rng, G=3, T=5)
    R, parts = block_scores(q, idx, threads=2, return_partials=True)
    assert np.allclose(parts.sum(axis=1), 3 * 5, rtol=1e-13)
    assert np.allclose(parts.sum(axis=0) / (2 * 6), R, rtol=1e-13)
    assert np.allclose(lg_partial_scores(q, idx, 1, 0), parts[2], rtol=0, atol=0)


def test_tiny_workspace_planted_block_ranks_first():
    wl = synth.get_workload("tiny")
    res = run_step(wl, threads=1)
    assert int(np.argmax(res["R"])) == wl.planted_block
    assert wl.planted_block in set(res["sel"].tolist())
    assert len(res["sel"]) == 11 and list(res["base_pos"]) == list(range(0, 352, 32))


# --------------------------------------------------- streamed (tiled) form ----
# KVMem Sec. 5: scoring an index that does not fit at once keeps the global
# softmax normalisation, so it equals Eq. (10) over the complete index.

from oracle.scores import block_scores_streamed  # noqa: E402


def _slicer(idx):
    return lambda l, g: idx[l, g]


def test_streamed_scores_equal_resident_scores():
    rng = np.random.default_rng(31)
    for (L, Hkv, G, T, N, d) in [(2, 2, 3, 4, 37, 16), (3, 1, 2, 5, 1, 8),
                                 (1, 4, 1, 1, 129, 32), (2, 3, 2, 3, 250, 8)]:
        q, idx = rand_case(rng, L=L, Hkv=Hkv, G=G, T=T, N=N, d=d)
        want = block_scores(q, idx, threads=1)
        got = block_scores_streamed(q, _slicer(idx), Hkv, N, threads=3)
        assert np.array_equal(got, want)
        assert abs(got.sum() - T) < 1e-12


def test_streamed_scores_catch_a_transposed_pair():
    # A planted mistake (the (l, g) slice of another pair) must change R.
    rng = np.random.default_rng(32)
    q, idx = rand_case(rng, L=2, Hkv=2, G=3, T=4, N=37, d=16)
    want = block_scores_streamed(q, _slicer(idx), 2, 37, threads=2)
    wrong = block_scores_streamed(q, lambda l, g: idx[1 - l, g], 2, 37, threads=2)
    assert np.max(np.abs(wrong - want)) > 1e-3
    wrong = block_scores_streamed(q, lambda l, g: idx[l, 1 - g], 2, 37, threads=2)
    assert np.max(np.abs(wrong - want)) > 1e-3


def test_streamed_constant_index_and_single_row():
    rng = np.random.default_rng(33)
    q = rng.standard_normal((2, 4, 3, 8))
    idx = np.broadcast_to(rng.standard_normal((2, 2, 1, 8)), (2, 2, 50, 8)).copy()
    assert np.allclose(block_scores_streamed(q, _slicer(idx), 2, 50), 3 / 50, rtol=0, atol=1e-15)
    q = rng.standard_normal((1, 1, 1, 32))
    idx = rng.standard_normal((1, 1, 200, 32)) * 3
    want = scipy.special.softmax(idx[0, 0] @ q[0, 0, 0] / math.sqrt(32))
    assert np.allclose(block_scores_streamed(q, _slicer(idx), 1, 200), want, rtol=1e-13, atol=0)
