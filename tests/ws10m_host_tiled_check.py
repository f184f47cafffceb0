"""The 10M-token host-tiled scoring check, run in a process of its own by
test_gpu_scale_fullsize.py (it pins 41 GB of host memory; the test suite's own
process never holds that memory and never creates a context after it).

KVMem Sec. 5: scoring with the index streamed from pinned host memory in 64 MiB
tiles (611 tiles at 10M tokens) keeps the global softmax, so it equals scoring
the resident index: bit-identical here, and within 1e-5 of the oracle's scores
(tests/golden/ws10m_oracle.npz). Prints one JSON line with what it checked;
exits non-zero on any failed check.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import attention_space_block_amd as k  # noqa: E402
import synth  # noqa: E402
from oracle import select_blocks  # noqa: E402
from tests import gpu_common as gc  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    assert torch.cuda.is_available()
    k._abi.lib()
    dev = torch.device("cuda:0")
    g = np.load(os.path.join(HERE, "golden", "ws10m_oracle.npz"))
    wl = synth.get_workload("ws10m")
    N, tb, d = wl.n_blocks, wl.tile_blocks, wl.head_dim
    nlg = wl.n_layers * wl.n_kv_heads
    ntile = (N + tb - 1) // tb
    say("ws10m: drawing the 41 GB index into pinned tiles")
    host = torch.empty((ntile, nlg, tb, d), dtype=torch.int16).pin_memory()
    hv = host.numpy().view(np.uint16)
    for t in range(ntile):
        nb = min(tb, N - t * tb)
        synth.index_direct(wl, t * tb, nb, out=hv[t], lg_stride_elems=tb * d)
    say("ws10m: device copy of the index")
    index = torch.empty((wl.n_layers, wl.n_kv_heads, N, d), dtype=torch.int16, device=dev)
    iv = index.view(nlg, N, d)
    for t in range(ntile):
        nb = min(tb, N - t * tb)
        iv[:, t * tb:t * tb + nb, :].copy_(host[t, :, :nb, :].to(dev, non_blocking=False))
    q = gc.to_dev(synth.query(wl), dev)
    say("ws10m: scoring, index in HBM")
    res = gc.score_dev(k, wl, q, index, N, N, dev).cpu().numpy()
    del index, iv
    say("ws10m: scoring, index streamed from pinned host tiles")
    til = gc.score_dev(k, wl, q, None, N, N, dev, loc=1, tile_blocks=tb, host_index=host)
    til = til.cpu().numpy()
    out = {"tiles": ntile, "bit_identical": bool(np.array_equal(res, til))}
    rel = np.abs(res.astype(np.float64) - g["R"]) / g["R"]
    out["max_rel_err"] = float(rel.max())
    out["margin"] = float(g["margin"])
    sel, n_sel, base = gc.select_dev(k, torch.from_numpy(res).to(dev), N, wl.n_sink,
                                     wl.n_recent, wl.budget_blocks, dev)
    n = int(n_sel.item())
    s = sel.cpu().numpy()[:n]
    out["n_sel"] = n
    out["selection_exact_on_gpu_scores"] = bool(np.array_equal(
        s, select_blocks(res.astype(np.float64), wl.n_sink, wl.n_recent, wl.budget_blocks)))
    out["selection_equals_oracle"] = (bool(np.array_equal(s, g["sel"]))
                                      if out["margin"] > 2e-5 else None)
    ok = (out["bit_identical"] and out["max_rel_err"] <= 1e-5 and n == wl.budget_blocks
          and out["selection_exact_on_gpu_scores"] and out["selection_equals_oracle"] is not False)
    if ok:
        gc.check_selection(s, g["R"], wl.n_sink, wl.n_recent, wl.budget_blocks)
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
