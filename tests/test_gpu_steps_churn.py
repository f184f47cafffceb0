"""GPU parity over consecutive agent steps (the step-churn workspace).

Each step appends 64 freshly prefilled blocks (indexed and registered as
resident), rescores with that step's queries, reselects and rematerializes the
view with page reuse (KVMem Sec. 4.4, Sec. 5). Checked per step:

- scores: sum R = T; against the oracle's Eq. (10) where it computed the step
  in full (every step of the 4-layer workspace; steps 0, 1, 16 and 31 of the
  64-layer one), and on the 64-layer workspace every step's sums of one
  (layer, KV head) pair drawn per step, scored through the same entry point
  on that pair's slices;
- selection: bit-exact against the oracle's selector on the GPU's own fp32
  scores at every step, and against the oracle's selection where its cutoff
  margin decides it;
- working-set delta: hits, misses and evictions against the oracle's bounded
  page-pool model (oracle.plan.PagePool, fed the same selections and
  registrations), and the resident set G_t against the library's records;
- page reuse: every hit keeps its page;
- K/V pages of sampled hits and misses against the oracle's re-RoPE and V.
"""
import os

import numpy as np
import pytest

import synth
from oracle import PagePool, select_blocks
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def say(*a):
    print(*a, flush=True)


def pair_sums_dev(k, wl, q, index, n_blocks, cap, l, g, dev):
    """G * R of the single (layer, KV head) pair (l, g), scored through
    kvm_score_blocks on that pair's slices of q and of the index: the sum over
    the pair's query rows of the per-row softmax over all blocks."""
    G = wl.group
    d1 = k.Dims(1, 1, G, wl.head_dim, wl.block_tokens)
    qs = q[l, g * G:(g + 1) * G]                      # [G][T][d], contiguous
    ix = index[l, g]                                  # [cap][d], contiguous
    T = q.shape[2]
    ws_b = k.kvm_score_ws_bytes(d1, k.KVM_BF16, T, n_blocks)
    import torch
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    out = torch.empty(n_blocks, dtype=torch.float32, device=dev)
    k.kvm_score_blocks(d1, k.KVM_BF16, qs, T, ix, cap, n_blocks, k.KVM_INDEX_DEVICE, 0, out, ws,
                       ws_b)
    return out.cpu().numpy().astype(np.float64) * G


def run_churn(name, kv_every=1, n_check=4):
    import torch
    import attention_space_block_amd as k
    path = os.path.join(HERE, "golden", f"{name}_oracle.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    g = np.load(path)
    full_steps = [int(t) for t in g["full_steps"]] if "full_steps" in g else None
    dev = torch.device("cuda:0")
    wl = synth.get_workload(name)
    Kb, B, T = wl.budget_blocks, wl.block_tokens, wl.n_q_tokens
    n_slots = Kb + wl.append_blocks + 64
    say(f"{name}: building the index of {wl.n_blocks} blocks")
    upd = k.WorkingSetUpdater(k.dims_for(wl), k.KVM_BF16, wl.final_blocks, Kb, wl.n_sink,
                              wl.n_recent, n_slots, (Kb + wl.reserve_blocks) * B, dev, wl.theta,
                              wl.rope_layout, batch_blocks=64, staging_blocks=256)
    upd.index.copy_(gc.build_index_streamed(k, wl, dev, n_blocks=wl.n_blocks,
                                            cap=wl.final_blocks))
    upd.n_blocks = wl.n_blocks
    fn, user, keep = synth.gather_store(wl)
    upd.ctx.kvm_ctx_set_gather_raw(0, wl.final_blocks, fn, user)
    model = PagePool(n_slots)
    rng = np.random.default_rng(5)
    page_of = {}                                  # block -> page while resident
    for t in range(wl.steps):
        if t > 0:
            b0 = upd.n_blocks
            nk = gc.raw_to_device(wl, "K", b0, wl.append_blocks, dev)
            nv = gc.raw_to_device(wl, "V", b0, wl.append_blocks, dev)
            upd.append(nk, nv, wl.append_blocks)
            torch.cuda.synchronize()
            for b in model.register(range(b0, b0 + wl.append_blocks)):
                page_of.pop(b, None)
            for b in range(b0, b0 + wl.append_blocks):
                page_of[b] = upd.ctx.kvm_ctx_block_state(b)[0]
        N = upd.n_blocks
        q = gc.to_dev(synth.query(wl, step=t), dev)
        st = upd.update(q, T)
        torch.cuda.synchronize()
        n = int(upd.n_sel.item())
        sel = upd.sel.cpu().numpy()[:n]
        say(f"step {t}: {st}")
        R = upd.scores.cpu().numpy()[:N].astype(np.float64)
        assert abs(R.sum() - T) <= 1e-5 * T
        # the selection is the oracle's selector applied to these fp32 scores
        assert np.array_equal(sel, select_blocks(R, wl.n_sink, wl.n_recent, Kb))
        if f"P_{t}" in g:
            l, gg = (int(x) for x in g[f"lg_{t}"])
            P = pair_sums_dev(k, wl, q, upd.index, N, upd.cap, l, gg, dev)
            rel = np.max(np.abs(P - g[f"P_{t}"]) / g[f"P_{t}"])
            say(f"  pair ({l}, {gg}) max rel err {rel:.2e}")
            assert rel <= 1e-5
        if full_steps is None or t in full_steps:
            j = t if full_steps is None else full_steps.index(t)
            Ro = g[f"R_{t}"]
            rel = np.max(np.abs(R - Ro) / Ro)
            say(f"  full scores max rel err {rel:.2e}, margin {g['margin'][j]:.2e}")
            assert rel <= 1e-5
            if g["margin"][j] > 2e-5:
                assert np.array_equal(sel, g["sel"][j])
            gc.check_selection(sel, Ro, wl.n_sink, wl.n_recent, Kb)
        # working-set delta against the oracle's page-pool model
        r = model.update(sel.tolist())
        assert st["hits"] == len(r["hits"]) and st["misses"] == len(r["misses"])
        assert st["evicted"] == len(r["evicted"])
        for b in r["evicted"]:
            page_of.pop(b, None)
        page = upd.page_table.cpu().numpy()[:n]
        assert len(set(page.tolist())) == n and page.min() >= 0 and page.max() < n_slots
        view = dict(zip(sel.tolist(), page.tolist()))
        for b in r["hits"]:
            assert view[b] == page_of[b]              # GPU hits keep their page in place
        page_of.update(view)
        lib_resident = {b for b in range(N) if upd.ctx.kvm_ctx_block_state(b)[0] >= 0}
        assert lib_resident == model.resident
        # K/V pages of sampled hits and misses
        if t % kv_every == 0:
            hits, misses = set(r["hits"]), set(r["misses"])
            miss_pos = [i for i, b in enumerate(sel) if b in misses]
            hit_pos = [i for i, b in enumerate(sel) if b in hits]
            check = sorted(
                set(rng.choice(miss_pos, min(n_check, len(miss_pos)), replace=False).tolist())
                | set(rng.choice(hit_pos, min(n_check, len(hit_pos)), replace=False).tolist()))
            pool = type("P", (), {"k_view": upd.k_view, "v_view": upd.v_view})
            gc.check_view(wl, sel, page, pool, blocks=check)
    upd.close()


@pytest.mark.timeout(900)
def test_churn_steps_match_oracle():
    """4 layers, 8 steps: every step checked in full."""
    run_churn("churn_l4")


@pytest.mark.timeout(1100)
def test_churn_full_size_32_steps():
    """The churn workspace at its stated size: 64 layers, 32 steps. K/V of
    sampled hits and misses are checked on every 4th step."""
    run_churn("churn", kv_every=4)
