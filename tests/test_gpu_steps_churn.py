"""GPU parity over consecutive agent steps (the step-churn workspace).

Each step appends 64 freshly prefilled blocks, rescoring and reselecting with
that step's queries, and rematerializes the view with page reuse. Checked per
step against the CPU oracle: the selection (tests/golden, when the oracle's
cutoff margin allows a decision), sampled scores, the working-set delta
(misses = W_t minus the resident set G_{t-1}, KVMem Sec. 4.4), page reuse for
retained blocks, and K/V pages of sampled blocks (hits and misses).
"""
import os

import numpy as np
import pytest

import synth
from oracle import working_set_delta
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(900)
def test_churn_steps_match_oracle():
    import torch
    import attention_space_block_amd as k
    path = os.path.join(HERE, "golden", "churn_l4_oracle.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path)
    dev = torch.device("cuda:0")
    wl = synth.get_workload("churn_l4")
    Kb, B, T = wl.budget_blocks, wl.block_tokens, wl.n_q_tokens
    upd = k.WorkingSetUpdater(k.dims_for(wl), k.KVM_BF16, wl.final_blocks, Kb, wl.n_sink,
                              wl.n_recent, Kb + wl.append_blocks + 64,
                              (Kb + wl.reserve_blocks) * B, dev, wl.theta, wl.rope_layout,
                              batch_blocks=64, staging_blocks=256)
    upd.index.copy_(gc.build_index_streamed(k, wl, dev, n_blocks=wl.n_blocks,
                                            cap=wl.final_blocks))
    upd.n_blocks = wl.n_blocks
    fn, user, keep = synth.gather_store(wl)
    upd.ctx.kvm_ctx_set_gather_raw(0, wl.final_blocks, fn, user)
    rng = np.random.default_rng(5)
    prev_view = {}
    for t in range(wl.steps):
        if t > 0:
            b0 = upd.n_blocks
            nk = gc.raw_to_device(wl, "K", b0, wl.append_blocks, dev)
            nv = gc.raw_to_device(wl, "V", b0, wl.append_blocks, dev)
            upd.append(nk, nv, wl.append_blocks)
            torch.cuda.synchronize()
        resident = {b for b in range(upd.n_blocks) if upd.ctx.kvm_ctx_block_state(b)[0] >= 0}
        q = gc.to_dev(synth.query(wl, step=t), dev)
        st = upd.update(q, T)
        torch.cuda.synchronize()
        n = int(upd.n_sel.item())
        sel = upd.sel.cpu().numpy()[:n]
        print(f"step {t}: {st}", flush=True)
        # scores and selection against the oracle
        R = upd.scores.cpu().numpy()[:upd.n_blocks].astype(np.float64)
        Ro = g[f"R_{t}"]
        assert np.max(np.abs(R - Ro) / Ro) <= 1e-5
        if g["margin"][t] > 2e-5:
            assert np.array_equal(sel, g["sel"][t])
        gc.check_selection(sel, Ro, wl.n_sink, wl.n_recent, Kb)
        # working-set delta against the resident set before the step
        delta = working_set_delta(set(prev_view), set(sel.tolist()), resident)
        assert st["misses"] == len(delta["physical_in"])
        assert st["hits"] == len(delta["hits"])
        page = upd.page_table.cpu().numpy()[:n]
        assert len(set(page.tolist())) == n
        view = dict(zip(sel.tolist(), page.tolist()))
        for b in delta["retained"]:
            assert view[b] == prev_view[b]          # GPU hits keep their page in place
        # K/V pages of sampled hits and misses
        miss_pos = [i for i, b in enumerate(sel) if b in delta["physical_in"]]
        hit_pos = [i for i, b in enumerate(sel) if b in delta["hits"]]
        check = sorted(set(rng.choice(miss_pos, min(4, len(miss_pos)), replace=False).tolist())
                       | set(rng.choice(hit_pos, min(4, len(hit_pos)), replace=False).tolist()))
        pool = type("P", (), {"k_view": upd.k_view, "v_view": upd.v_view})
        gc.check_view(wl, sel, page, pool, blocks=check)
        prev_view = view
    upd.close()
