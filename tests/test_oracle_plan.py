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
