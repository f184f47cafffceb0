"""Parity of the library's host-tier simulator (kvm_tier_simulate, KVMem Sec. 4.4
hierarchical reuse) with the oracle: integer outputs, compared exactly. The call is
host code of libkvm; it runs with the GPU tests because it goes through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import simulate_host_tier

pytestmark = pytest.mark.gpu

POLICIES = [("lru", 0.0), ("lrfu", 0.0), ("lrfu", 0.05), ("lrfu", 0.3), ("lrfu", 1.0)]


def _lib():
    import attention_space_block_amd as k
    return k


def _code(k, pol):
    return k.KVM_TIER_LRU if pol == "lru" else k.KVM_TIER_LRFU


def _random_trace(seed, n_steps, n_blocks, max_sel, p_miss):
    rng = np.random.default_rng(seed)
    steps, nxt = [], n_blocks
    for _ in range(n_steps):
        new = list(range(nxt, nxt + int(rng.integers(0, 4))))
        nxt += len(new)
        sel = sorted(set(rng.integers(0, nxt, size=int(rng.integers(1, max_sel))).tolist()))
        miss = [b for b in sel if rng.random() < p_miss]
        steps.append((new, sel, miss))
    return steps


@pytest.mark.parametrize("seed", range(6))
def test_tier_random_traces_match_oracle(seed):
    k = _lib()
    steps = _random_trace(seed, 80, 300 + 200 * seed, 60, 0.4)
    for cap in (1, 17, 150):
        for pol, lam in POLICIES:
            want = simulate_host_tier(steps, cap, pol, lam)
            got = k.kvm_tier_simulate(_code(k, pol), cap, lam, steps)
            assert got == want, (cap, pol, lam)


def test_tier_churn_selections_match_oracle():
    """The 4-layer churn workspace's per-step selections (from the oracle's
    expected values): misses are the selected blocks outside the previous
    selection and the step's new blocks."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "churn_l4_oracle.npz")
    g = np.load(path)
    wl = synth.get_workload("churn_l4")
    steps, prev = [], set()
    for t in range(wl.steps):
        new = [] if t == 0 else list(range(wl.n_blocks + (t - 1) * wl.append_blocks,
                                           wl.n_blocks + t * wl.append_blocks))
        sel = g["sel"][t].tolist()
        miss = [b for b in sel if b not in prev and b not in new]
        steps.append((new, sel, miss))
        prev = set(sel)
    k = _lib()
    for cap in (3000, 5000):
        for pol, lam in (("lru", 0.0), ("lrfu", 0.05), ("lrfu", 0.3)):
            assert k.kvm_tier_simulate(_code(k, pol), cap, lam, steps) == \
                simulate_host_tier(steps, cap, pol, lam)


def test_tier_error_paths():
    k = _lib()
    with pytest.raises(k.KvmError) as e:
        k.kvm_tier_simulate(k.KVM_TIER_LRU, 4, 0.0, [([], [3, 2], [])])     # not ascending
    assert e.value.code == k.api._abi.KVM_EINVAL
    with pytest.raises(k.KvmError) as e:
        k.kvm_tier_simulate(k.KVM_TIER_LRU, 4, 0.0, [([], [1, 2], [5])])    # miss not selected
    assert e.value.code == k.api._abi.KVM_EINVAL
    with pytest.raises(k.KvmError):
        k.kvm_tier_simulate(k.KVM_TIER_LRFU, 0, 0.1, [([], [1], [1])])      # no capacity
    with pytest.raises(k.KvmError):
        k.kvm_tier_simulate(k.KVM_TIER_LRFU, 4, -1.0, [([], [1], [1])])     # negative decay
    assert k.kvm_tier_simulate(k.KVM_TIER_LRU, 4, 0.0, []) == []
