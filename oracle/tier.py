"""Host-tier admission and eviction over a trace of agent steps.

KVMem Sec. 4.4 (hierarchical reuse): blocks evicted from the GPU pool are
reloaded from host memory when they are there and from NVMe otherwise; host
memory is bounded, and its admission and eviction weigh both recent retrieval
and cumulative retrieval frequency, against a recency-only baseline (LRU).

Reading (the pages give no formula): the recency-and-frequency weighting is
LRFU (Lee et al., "LRFU: A Spectrum of Policies that Subsumes the Least
Recently Used and Least Frequently Used Policies", IEEE Trans. Computers,
2001). A block touched at times t_1 < ... < t_k has combined value
CRF(t) = sum_i 2^(-lam * (t - t_i)); it is kept incrementally as
crf <- 1 + 2^(-lam * (t - t_last)) * crf. Since every value decays by the same
factor, the block with the smallest current value is the one with the
smallest key log2(crf) + lam * t_last, which does not change with t. lam = 0
gives LFU, lam = 1 gives LRU order. The LRU baseline uses key t_last.

Trace semantics, per step t (1-based), each list in ascending block order:
  1. new[t]: freshly prefilled blocks, staged out to host (admitted, touched);
  2. sel[t]: the step's selection: every selected block is touched (retrieval
     statistics are kept for every block, resident on the host or not);
  3. miss[t]: selected blocks that the GPU pool does not hold: a host copy is
     a host hit, otherwise the block is read from NVMe and admitted.
A block is touched at most once per step. Admission into a full host tier
first evicts (demotes to NVMe) the host block with the smallest key, the
lowest block id on ties. Returns per step (host_hits, nvme_reads, demotions).
"""
from __future__ import annotations

import math


def simulate_host_tier(steps, host_blocks: int, policy: str, lam: float = 0.0):
    """steps: list of (new, sel, miss) block lists; policy "lru" or "lrfu"."""
    assert host_blocks >= 1 and policy in ("lru", "lrfu")
    last, crf, key = {}, {}, {}
    host = set()
    out = []

    def touch(b, t):
        if last.get(b) == t:
            return
        if policy == "lrfu":
            prev = crf.get(b)
            crf[b] = 1.0 if prev is None else 1.0 + 2.0 ** (-lam * (t - last[b])) * prev
        last[b] = t
        key[b] = t if policy == "lru" else math.log2(crf[b]) + lam * t

    def admit(b):
        demoted = 0
        if b in host:
            return 0
        if len(host) >= host_blocks:
            victim = min(host, key=lambda x: (key[x], x))
            host.remove(victim)
            demoted = 1
        host.add(b)
        return demoted

    for t, (new, sel, miss) in enumerate(steps, start=1):
        dem = hits = nvme = 0
        for b in new:
            touch(b, t)
            dem += admit(b)
        for b in sel:
            touch(b, t)
        for b in miss:
            if b in host:
                hits += 1
            else:
                nvme += 1
                dem += admit(b)
        out.append((hits, nvme, dem))
    return out
