"""Write the oracle's expected values for the full-size workspaces.

Calls only the CPU oracle (which draws its inputs from the seeded generator).
Usage: python tests/golden/make_golden.py ws1m|ws10m|churn [threads]
Outputs tests/golden/<name>_oracle.npz.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import pipeline as op  # noqa: E402
from oracle.scores import block_scores, block_scores_streamed, lg_partial_scores  # noqa: E402
from oracle.select import select_blocks, cutoff_margin  # noqa: E402
from oracle.numerics import bf16_bits  # noqa: E402


# Steps of the full-size churn run whose scores the oracle computes in full.
FULL_CHURN_STEPS = (0, 1, 16, 31)


def churn_pair(wl, step):
    """The (layer, KV head) pair whose sums are kept for churn step `step`."""
    rng = np.random.default_rng(1000 + step)
    return int(rng.integers(wl.n_layers)), int(rng.integers(wl.n_kv_heads))


def one_step(wl, index, step, threads):
    q = op.query_f64(wl, step, index).astype(np.float32)       # exact bf16 values
    R = block_scores(q, index, threads=threads)
    sel = select_blocks(R, wl.n_sink, wl.n_recent, wl.budget_blocks)
    return R, sel, cutoff_margin(R, wl.n_sink, wl.n_recent, wl.budget_blocks)


def main():
    name = sys.argv[1]
    threads = int(sys.argv[2]) if len(sys.argv) > 2 else 8
    wl = synth.get_workload(name)
    t0 = time.time()
    out = {}
    if name == "ws10m":
        # the 41 GB index is drawn one (layer, KV head) slice at a time
        q = op.query_f64(wl, 0)
        Hkv = wl.n_kv_heads

        def slice_fn(l, g):
            return op.as_f64(synth.index_direct(wl, 0, wl.n_blocks, lg0=l * Hkv + g, n_lg=1,
                                                nthreads=2)[0], "bf16")
        R = block_scores_streamed(q, slice_fn, Hkv, wl.n_blocks, threads=threads)
        sel = select_blocks(R, wl.n_sink, wl.n_recent, wl.budget_blocks)
        out.update(R=R, sel=sel,
                   margin=np.float64(cutoff_margin(R, wl.n_sink, wl.n_recent, wl.budget_blocks)))
    elif name == "ws1m":
        index = op.index_rows(wl, 0, wl.n_blocks, threads=threads, out_dtype=np.float32)
        print(f"index {time.time() - t0:.0f}s", flush=True)
        R, sel, margin = one_step(wl, index, 0, threads)
        out.update(R=R, sel=sel.astype(np.int32), margin=np.float64(margin))
        # Mean-K of a few sampled blocks (bf16 bit patterns), for the full-size build check
        rng = np.random.default_rng(7)
        blocks = np.sort(rng.choice(wl.n_blocks, 4, replace=False))
        out.update(sample_blocks=blocks, sample_index_bits=bf16_bits(index[:, :, blocks, :]))
    elif name.startswith("churn"):
        # append the step's blocks, score with the step's queries
        N_end = wl.final_blocks
        index = op.index_rows(wl, 0, N_end, threads=threads, out_dtype=np.float32)
        print(f"index {time.time() - t0:.0f}s", flush=True)
        # The reduced workspace gets every step in full. The full-size one gets
        # every step's sums for one (layer, KV head) pair drawn per step, and
        # the whole of Eq. (10) at a few steps (a full step is about ten CPU
        # minutes here).
        full_steps = range(wl.steps) if wl.n_layers <= 4 else FULL_CHURN_STEPS
        sels, margins, Rs = {}, {}, {}
        for t in range(wl.steps):
            N = wl.n_blocks + t * wl.append_blocks
            if wl.n_layers > 4:
                l, g = churn_pair(wl, t)
                q = op.query_f64(wl, t, index).astype(np.float32)
                out[f"P_{t}"] = lg_partial_scores(q, index[:, :, :N, :], l, g)
                out[f"lg_{t}"] = np.array([l, g], dtype=np.int32)
            if t in full_steps:
                R, sel, margin = one_step(wl, index[:, :, :N, :], t, threads)
                sels[t], margins[t], Rs[t] = sel.astype(np.int32), margin, R
            print(f"step {t}: {time.time() - t0:.0f}s", flush=True)
        # scores of step t are R_<t> (lengths grow by the appended blocks)
        steps = sorted(Rs)
        out.update(full_steps=np.array(steps, dtype=np.int32),
                   sel=np.stack([sels[t] for t in steps]),
                   margin=np.array([margins[t] for t in steps]),
                   **{f"R_{t}": Rs[t] for t in steps})
    print(f"done {time.time() - t0:.0f}s", flush=True)
    np.savez_compressed(os.path.join(HERE, f"{name}_oracle.npz"), **out)


if __name__ == "__main__":
    main()
