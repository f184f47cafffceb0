"""Query-conditioned block relevance.

KVMem paper, Sec. 4.3, "Query-Conditioned Block Scoring" and Eq. (10) (the
displayed equation was lost; this is the reading of the prose around it):

  for every scored layer l, current query token m and query head h, the
  position-independent query q[l,m,h] is compared with the Mean-K vector of
  every candidate block b of the head's KV group g(h) by a scaled dot
  product s = q . kbar[l,b,g(h)] / sqrt(d); a softmax over the candidate
  blocks normalises each fixed (l,m,h); the normalised values are summed over
  the query tokens m and averaged over the L*Hq scored layer-head pairs:

      R_b = 1/(L*Hq) * sum_l sum_h sum_m softmax_b(s[l,m,h,:])_b

Readings: the candidate set is every indexed block (sink and recent blocks
take part in the softmax; they are only exempt from the top-k competition,
Sec. 5 tiled scoring "over the complete historical index"); g(h) = h // G
with G = Hq/Hkv (grouped-query attention); d is the head dimension.
Consequence used as a pin: sum_b R_b = T (the number of query tokens).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def pair_softmax_sums(rows: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Column sums over the query rows of one (layer, KV head) of the row-wise
    softmax of rows . kbar^T / sqrt(d). rows: [G*T][d]; kbar: [N][d]."""
    rows = np.asarray(rows, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    d = rows.shape[1]
    s = rows @ kbar.T / np.sqrt(d)                          # [G*T][N]
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)                    # softmax over blocks, per row
    return p.sum(axis=0)


def lg_partial_scores(q: np.ndarray, index: np.ndarray, l: int, g: int) -> np.ndarray:
    """sum over (m, h in group g) of softmax_b(q[l,h,m] . kbar[l,g,b] / sqrt(d)).

    q: [L][Hq][T][d]; index: [L][Hkv][N][d]. Returns [N]."""
    L, Hq, T, d = q.shape
    Hkv = index.shape[1]
    G = Hq // Hkv
    # query heads h with h // G == g share KV head g
    return pair_softmax_sums(q[l, g * G:(g + 1) * G].reshape(G * T, d), index[l, g])


def block_scores(q: np.ndarray, index: np.ndarray, threads: int | None = None,
                 return_partials: bool = False):
    """R[N] for all blocks; optionally also the [L*Hkv][N] per-(l,g) sums.

    q and index may be float32 arrays holding exact bf16/fp32 values; each
    (l, g) slice is widened to float64 before use."""
    L, Hq, T, d = q.shape
    Lx, Hkv, N, dx = index.shape
    if Lx != L or dx != d or Hq % Hkv:
        raise ValueError("shape mismatch")
    pairs = [(l, g) for l in range(L) for g in range(Hkv)]
    threads = threads or min(16, os.cpu_count() or 1)
    if threads > 1 and len(pairs) > 1:
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda lg: lg_partial_scores(q, index, *lg), pairs))
    else:
        parts = [lg_partial_scores(q, index, l, g) for (l, g) in pairs]
    total = np.zeros(N)
    for p in parts:
        total += p
    R = total / (L * Hq)
    if return_partials:
        return R, np.stack(parts)
    return R



def block_scores_streamed(q: np.ndarray, index_slice, n_kv_heads: int, n_blocks: int,
                          threads: int | None = None) -> np.ndarray:
    """The same R[N] as block_scores, for indexes too large to hold at once:
    index_slice(l, g) returns the [N][d] Mean-K rows of one (layer, KV head);
    each pair's softmax sums are formed exactly as in lg_partial_scores and the
    pairs are added in the same (l, g) order."""
    L, Hq, T, d = q.shape
    G = Hq // n_kv_heads
    pairs = [(l, g) for l in range(L) for g in range(n_kv_heads)]

    def one(lg):
        l, g = lg
        return pair_softmax_sums(q[l, g * G:(g + 1) * G].reshape(G * T, d), index_slice(l, g))

    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(one, pairs))
    total = np.zeros(n_blocks)
    for p in parts:
        total += p
    return total / (L * Hq)
