"""Pins of the working-set delta (KVMem paper Sec. 4.4)."""
import numpy as np

from oracle import working_set_delta


def test_set_identities_random():
    rng = np.random.default_rng(16)
    for _ in range(50):
        W0 = set(rng.choice(200, 60, replace=False).tolist())
        W1 = set(rng.choice(200, 60, replace=False).tolist())
        extra = set(rng.choice(200, 20, replace=False).tolist())
        G0 = W0 | extra
        d = working_set_delta(W0, W1, G0)
        assert d["retained"] | d["incoming"] == W1
        assert d["retained"] | d["outgoing"] == W0
        assert not (d["retained"] & d["incoming"]) and not (d["retained"] & d["outgoing"])
        assert d["hits"] | d["physical_in"] == W1 and not (d["hits"] & d["physical_in"])
        assert len(d["physical_in"]) == len(W1) - len(d["hits"])
        assert d["physical_in"] <= d["incoming"]


def test_pool_equal_to_previous_set_loads_exactly_the_incoming():
    d = working_set_delta({1, 2, 3}, {2, 3, 4, 5}, {1, 2, 3})
    assert d["physical_in"] == {4, 5} == d["incoming"]
    assert d["outgoing"] == {1} and d["retained"] == {2, 3}


# ------------------------------------------------------- bounded page pool ----
import pytest  # noqa: E402

from oracle.plan import PagePool, PoolFull  # noqa: E402


def test_pool_hand_trace_lru_outside_the_view():
    p = PagePool(4)
    r = p.update([1, 2, 3])                       # step 1: three cold misses
    assert r["hits"] == [] and r["misses"] == [1, 2, 3] and r["evicted"] == []
    r = p.update([2, 3, 4])                       # step 2: one free page left
    assert r["hits"] == [2, 3] and r["misses"] == [4] and r["evicted"] == []
    assert p.resident == {1, 2, 3, 4}
    r = p.update([3, 5, 6])                       # step 3: 1 (step 1) goes, then 2 (step 2)
    assert r["hits"] == [3] and r["misses"] == [5, 6] and r["evicted"] == [1, 2]
    assert p.resident == {3, 4, 5, 6}
    r = p.update([4, 7])                          # step 4
    # last uses: 3 -> 3, 4 -> 2, 5 -> 3, 6 -> 3; 4 is selected, so 3 (tie at 3, lowest id)
    assert r["hits"] == [4] and r["misses"] == [7] and r["evicted"] == [3]
    assert p.resident == {4, 5, 6, 7}


def test_pool_ties_go_to_the_lower_block_id():
    p = PagePool(3)
    p.update([10, 20, 30])
    r = p.update([40, 50])
    assert r["evicted"] == [10, 20] and p.resident == {30, 40, 50}


def test_pool_registered_blocks_are_protected_until_the_next_update():
    p = PagePool(4)
    p.update([1, 2, 3])
    assert p.register([9]) == []                  # a free page
    with pytest.raises(PoolFull):
        p.register([10])                          # 1, 2, 3 and 9 are all current
    assert p.resident == {1, 2, 3, 9}
    r = p.update([1, 9])                          # 2 and 3 fall out of the view
    assert r["hits"] == [1, 9] and r["misses"] == [] and r["evicted"] == []
    assert p.register([10, 11]) == [2, 3]
    with pytest.raises(PoolFull):                 # all or nothing
        p.register([12, 13])
    assert p.resident == {1, 9, 10, 11}
    r = p.update([10, 12])
    # last uses: 1 -> 2, 9 -> 2, 10 -> 2, 11 -> 2: ties at step 2, lowest id first
    assert r["hits"] == [10] and r["misses"] == [12] and r["evicted"] == [1]


def test_pool_view_larger_than_pool_is_refused():
    with pytest.raises(PoolFull):
        PagePool(2).update([1, 2, 3])


def test_pool_invariants_and_delta_on_random_traces():
    rng = np.random.default_rng(17)
    for trial in range(30):
        cap = int(rng.integers(5, 40))
        p = PagePool(cap)
        W_prev = set()
        nb = 20
        for t in range(25):
            if rng.random() < 0.5:
                new = list(range(nb, nb + int(rng.integers(1, 4))))
                nb += len(new)
                before = p.resident
                try:
                    ev = p.register(new)
                except PoolFull:
                    assert p.resident == before
                else:
                    assert set(new) <= p.resident and not (set(ev) & set(new))
                    assert p.resident == (before | set(new)) - set(ev)
            k = int(rng.integers(1, cap + 1))
            W = set(rng.choice(nb, min(k, nb), replace=False).tolist())
            G_prev = p.resident
            r = p.update(W)
            d = working_set_delta(W_prev, W, G_prev)
            assert set(r["hits"]) == d["hits"] and set(r["misses"]) == d["physical_in"]
            assert set(r["evicted"]) <= G_prev - W
            assert p.resident == (G_prev | W) - set(r["evicted"])
            assert len(p.resident) <= cap and W <= p.resident
            # evictions happen only when the pool would overflow
            assert len(r["evicted"]) == max(0, len(G_prev) + len(r["misses"]) - cap)
            W_prev = W


def test_pool_as_large_as_every_block_never_evicts():
    rng = np.random.default_rng(18)
    p = PagePool(100)
    seen = set()
    for t in range(20):
        W = set(rng.choice(100, 30, replace=False).tolist())
        r = p.update(W)
        assert r["evicted"] == [] and set(r["misses"]) == W - seen
        seen |= W
        assert p.resident == seen


def test_pool_exactly_the_view_size_holds_the_previous_view():
    # with no registrations and a pool of |W| pages, G_{t-1} = W_{t-1}, so the
    # physical loads are exactly the incoming set L_t
    rng = np.random.default_rng(19)
    p = PagePool(12)
    W_prev = set()
    for t in range(15):
        W = set(rng.choice(40, 12, replace=False).tolist())
        r = p.update(W)
        assert set(r["misses"]) == W - W_prev and set(r["evicted"]) == (W_prev - W)
        assert p.resident == W
        W_prev = W
