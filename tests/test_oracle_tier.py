"""Pins of host-tier admission and eviction (KVMem Sec. 4.4, hierarchical reuse;
LRFU of Lee et al. 2001 as the recency-and-frequency policy)."""
import numpy as np

from oracle import simulate_host_tier

A, B, C = 10, 20, 30
# A is retrieved three steps in a row, then the GPU loses it while B and C are
# fetched; with two host slots, LRU demotes A (least recent) and must read it
# from NVMe again, LRFU keeps A (frequently retrieved) and demotes B.
HAND = [([], [A], [A]), ([], [A], []), ([], [A], []), ([], [B], [B]), ([], [C], [C]),
        ([], [A], [A])]


def test_hand_trace_lru_demotes_the_frequent_block():
    got = simulate_host_tier(HAND, 2, "lru")
    assert got == [(0, 1, 0), (0, 0, 0), (0, 0, 0), (0, 1, 0), (0, 1, 1), (0, 1, 1)]


def test_hand_trace_lrfu_keeps_the_frequent_block():
    # keys at step 5: A = log2(1 + 2^-.1 (1 + 2^-.1)) + .1*3 = 1.79, B = .4
    got = simulate_host_tier(HAND, 2, "lrfu", 0.1)
    assert got == [(0, 1, 0), (0, 0, 0), (0, 0, 0), (0, 1, 0), (0, 1, 1), (1, 0, 0)]


def test_lambda_zero_is_lfu():
    # B touched twice, A once but later: LFU demotes A when C arrives
    steps = [([], [B], [B]), ([], [B], []), ([], [A], [A]), ([], [C], [C]), ([], [A, B], [A, B])]
    got = simulate_host_tier(steps, 2, "lrfu", 0.0)
    assert got[3] == (0, 1, 1)
    assert got[4] == (1, 1, 1)      # B is a host hit, A comes back from NVMe


def _random_trace(seed, n_steps=60, n_blocks=40, one_touch=False):
    rng = np.random.default_rng(seed)
    steps, nxt = [], n_blocks
    for _ in range(n_steps):
        new = [] if one_touch or rng.random() < 0.6 else [nxt + i for i in range(rng.integers(1, 4))]
        nxt += len(new)
        if one_touch:
            sel = [int(rng.integers(0, n_blocks))]
        else:
            sel = sorted(set(rng.integers(0, nxt, size=rng.integers(1, 12)).tolist()))
        miss = [b for b in sel if rng.random() < 0.5]
        steps.append((new, sel, miss))
    return steps


def test_lambda_one_orders_like_lru_when_touch_times_are_distinct():
    for seed in range(20):
        steps = _random_trace(seed, one_touch=True)
        assert simulate_host_tier(steps, 5, "lrfu", 1.0) == simulate_host_tier(steps, 5, "lru")


def test_conservation_and_capacity():
    """hits + NVMe reads = misses each step; the host only grows until full and
    then demotes one block per insertion, so cumulative demotions equal
    max(0, cumulative insertions - capacity) (new blocks are fresh ids here)."""
    for seed in range(10):
        steps = _random_trace(100 + seed)
        for pol, lam in (("lru", 0.0), ("lrfu", 0.05), ("lrfu", 0.5)):
            out = simulate_host_tier(steps, 7, pol, lam)
            ins = dem = 0
            for (new, sel, miss), (hits, nvme, d) in zip(steps, out):
                assert hits + nvme == len(miss)
                ins += len(new) + nvme
                dem += d
                assert dem == max(0, ins - 7)


def test_unbounded_host_reads_each_block_from_nvme_at_most_once():
    for seed in range(10):
        steps = _random_trace(200 + seed)
        out = simulate_host_tier(steps, 10**6, "lrfu", 0.2)
        staged = set()
        want = []
        for new, sel, miss in steps:
            staged.update(new)
            n = 0
            for b in miss:
                if b not in staged:
                    n += 1
                    staged.add(b)
            want.append(n)
        assert [o[1] for o in out] == want
        assert all(o[2] == 0 for o in out)
