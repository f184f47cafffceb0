"""Pins of the selector and compact positions (KVMem paper Sec. 4.3, 4.4, 5)."""
import itertools

import numpy as np
import pytest

import synth
from oracle import select_blocks, compact_positions, cutoff_margin


def brute_rank(R, n_sink, n_recent, budget):
    """O(N^2): candidate b is kept iff fewer than k candidates beat it, where c
    beats b when R_c > R_b, or R_c == R_b and c < b."""
    N = len(R)
    if N <= budget:
        return list(range(N))
    cand = range(n_sink, N - n_recent)
    k = budget - n_sink - n_recent
    keep = [b for b in cand
            if sum(1 for c in cand if R[c] > R[b] or (R[c] == R[b] and c < b)) < k]
    return sorted(set(range(n_sink)) | set(range(N - n_recent, N)) | set(keep))


def test_matches_rank_definition_with_many_ties():
    for seed in range(30):
        n = 20 + seed
        R = synth.scores_f32(seed, n, kind="ties", levels=3)
        for (s, r, bud) in [(1, 2, 11), (0, 0, 5), (2, 3, 5), (1, 1, n - 1)]:
            assert select_blocks(R, s, r, bud).tolist() == brute_rank(R, s, r, bud)


def test_exhaustive_subsets_unique_dominating_choice():
    rng = np.random.default_rng(10)
    for _ in range(40):
        N = int(rng.integers(4, 11))
        R = rng.integers(0, 3, N).astype(np.float32)       # heavy ties
        s, r = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        budget = int(rng.integers(s + r, N))
        cand = list(range(s, N - r))
        k = budget - s - r

        def beats(c, b):
            return R[c] > R[b] or (R[c] == R[b] and c < b)
        dominating = [set(S) for S in itertools.combinations(cand, k)
                      if all(beats(x, y) for x in S for y in cand if y not in S)]
        assert len(dominating) == 1
        want = sorted(set(range(s)) | set(range(N - r, N)) | dominating[0])
        assert select_blocks(R, s, r, budget).tolist() == want


def test_shape_order_forced_and_small_history():
    R = synth.scores_f32(3, 500)
    sel = select_blocks(R, 1, 64, 200)
    assert len(sel) == 200 and np.all(np.diff(sel) > 0)
    assert 0 in sel and set(range(436, 500)) <= set(sel.tolist())
    assert select_blocks(R[:100], 1, 64, 200).tolist() == list(range(100))
    assert select_blocks(R[:200], 1, 64, 200).tolist() == list(range(200))


def test_top_k_are_the_largest_candidates():
    R = synth.scores_f32(4, 1000)
    sel = set(select_blocks(R, 1, 10, 60).tolist())
    cand = np.arange(1, 990)
    kept = [b for b in cand if b in sel]
    dropped = [b for b in cand if b not in sel]
    assert len(kept) == 49 and min(R[kept]) >= max(R[dropped])


def test_error_paths():
    R = synth.scores_f32(5, 50)
    with pytest.raises(ValueError):
        select_blocks(R, 5, 5, 9)
    bad = R.copy()
    bad[3] = np.nan
    with pytest.raises(ValueError):
        select_blocks(bad, 1, 1, 10)
    bad[3] = -1.0
    with pytest.raises(ValueError):
        select_blocks(bad, 1, 1, 10)


def test_compact_positions_closed_form():
    assert compact_positions(11).tolist() == [32 * i for i in range(11)]
    assert compact_positions(3, 16).tolist() == [0, 16, 32]


def test_cutoff_margin():
    R = np.array([9.0, 4.0, 2.0, 1.0, 3.0, 0.5])
    # sink 1, recent 1, budget 4 -> k = 2 among [4, 2, 1, 3]: kept 4, 3; next 2
    assert cutoff_margin(R, 1, 1, 4) == pytest.approx((3.0 - 2.0) / 3.0)
    assert cutoff_margin(R, 1, 1, 6) == float("inf")


def test_band_selection_check_accepts_exact_and_rejects_wrong_choices():
    from tests.gpu_common import check_selection
    R = synth.scores_f32(77, 3000).astype(np.float64)
    sel = select_blocks(R, 1, 64, 500)
    check_selection(sel, R, 1, 64, 500)                     # the oracle's own choice
    cand = [b for b in range(1, 3000 - 64) if b not in set(sel.tolist())]
    worst_in = min((b for b in sel if 1 <= b < 3000 - 64), key=lambda b: R[b])
    best_out = max(cand, key=lambda b: R[b])
    swapped = np.sort(np.r_[sel[sel != worst_in], best_out])
    # swapping the boundary pair is allowed only inside the band
    rel_gap = (R[worst_in] - R[best_out]) / R[worst_in]
    if rel_gap > 4e-5:
        with pytest.raises(AssertionError):
            check_selection(swapped, R, 1, 64, 500)
    far_out = min(cand, key=lambda b: R[b])
    bad = np.sort(np.r_[sel[sel != worst_in], far_out])
    with pytest.raises(AssertionError):
        check_selection(bad, R, 1, 64, 500)
    with pytest.raises(AssertionError):
        check_selection(sel[1:], R, 1, 64, 500)             # missing sink / wrong count
