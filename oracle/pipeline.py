"""The oracle run end to end on one seeded synthetic workspace.

Inputs come from ``synth`` (the only code shared with the HIP side); every
step of the method is one of this package's functions, in the order of the
KVMem paper's step-level lifecycle (Sec. 4.2-4.4): Mean-K index, block
relevance, selection, compact positions, re-RoPE of raw K and verbatim V.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import synth
from .meank import mean_k
from .numerics import from_bf16_bits, fp8_decode
from .rope import rope_rotate
from .scores import block_scores
from .select import select_blocks, compact_positions, cutoff_margin


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return from_bf16_bits(a)
    if dtype == "fp8":
        return fp8_decode(a)
    return np.asarray(a, dtype=np.float64)


def raw_blocks(wl, which: str, b0: int, nb: int) -> np.ndarray:
    """Raw K or V of blocks [b0, b0+nb) as float64 [nb][L][Hkv][B][d]."""
    return as_f64(synth.kv_blocks(wl, which, b0, nb), wl.dtype)


def index_rows(wl, b0: int, nb: int, chunk: int = 64, threads: int | None = None,
               out_dtype=np.float64) -> np.ndarray:
    """Stored Mean-K of blocks [b0, b0+nb) as [L][Hkv][nb][d].

    The stored values are bf16 or fp32 numbers, so out_dtype=np.float32 holds
    them exactly at half the memory of float64."""
    L, Hkv, d = wl.n_layers, wl.n_kv_heads, wl.head_dim
    out = np.empty((L, Hkv, nb, d), dtype=out_dtype)
    if wl.index_direct:
        return as_f64(synth.index_direct(wl, b0, nb), "bf16").astype(out_dtype)
    starts = list(range(0, nb, chunk))

    def work(s):
        n = min(chunk, nb - s)
        m = mean_k(raw_blocks(wl, "K", b0 + s, n), wl.index_dtype)    # [n][L][Hkv][d]
        out[:, :, s:s + n, :] = np.transpose(m, (1, 2, 0, 3))

    threads = threads or min(16, os.cpu_count() or 1)
    if threads > 1 and len(starts) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, starts))
    else:
        for s in starts:
            work(s)
    return out


def planted_shift(wl, index: np.ndarray) -> np.ndarray:
    """Tiny workspace: gain * Mean-K of the planted block, per query head's group,
    as the fp32 shift added to every query token."""
    L, Hq, d, G = wl.n_layers, wl.n_q_heads, wl.head_dim, wl.group
    sh = np.empty((L, Hq, d), dtype=np.float32)
    for l in range(L):
        for h in range(Hq):
            sh[l, h] = (wl.planted_gain * index[l, h // G, wl.planted_block]).astype(np.float32)
    return sh


def query_f64(wl, step: int = 0, index: np.ndarray | None = None) -> np.ndarray:
    shift = None
    if wl.planted_block >= 0:
        shift = planted_shift(wl, index)
    return as_f64(synth.query(wl, step=step, shift=shift), wl.index_dtype)


def query_stored(wl, step: int = 0, index: np.ndarray | None = None) -> np.ndarray:
    """The query exactly as handed to the library (bf16 bits or fp32)."""
    shift = planted_shift(wl, index) if wl.planted_block >= 0 else None
    return synth.query(wl, step=step, shift=shift)


def run_step(wl, n_blocks: int | None = None, step: int = 0, index: np.ndarray | None = None,
             threads: int | None = None) -> dict:
    """Index (unless given), scores, selection and positions for one step."""
    N = n_blocks if n_blocks is not None else wl.n_blocks
    if index is None:
        index = index_rows(wl, 0, N)
    q = query_f64(wl, step, index)
    R, parts = block_scores(q, index, threads=threads, return_partials=True)
    sel = select_blocks(R, wl.n_sink, wl.n_recent, wl.budget_blocks)
    return {
        "index": index,
        "q": q,
        "R": R,
        "partials": parts,
        "sel": sel,
        "base_pos": compact_positions(len(sel), wl.block_tokens),
        "margin": cutoff_margin(R, wl.n_sink, wl.n_recent, wl.budget_blocks),
    }


def expected_view_k(wl, block: int, base_pos: int) -> np.ndarray:
    """K of one block re-encoded at compact positions base_pos .. base_pos+B-1,
    float64 unrounded, [L][Hkv][B][d]."""
    k = raw_blocks(wl, "K", block, 1)[0]
    pos = base_pos + np.arange(wl.block_tokens)
    return rope_rotate(k, pos, wl.theta, wl.rope_layout)


def expected_view_v_bits(wl, block: int) -> np.ndarray:
    """V of one block exactly as stored (bit pattern), [L][Hkv][B][d]."""
    return synth.kv_blocks(wl, "V", block, 1)[0]
