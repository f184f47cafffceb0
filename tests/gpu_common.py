"""Helpers shared by the GPU tests: run the library on a seeded workspace.

Inputs come from ``synth``; every computed value comes from the HIP library
through its C ABI (``attention_space_block_amd``); expected values come from
``oracle``.
"""
from __future__ import annotations

import numpy as np

import synth


def torch_dtype(wl):
    """torch dtype holding the workspace's raw K/V and page elements."""
    import torch
    return {"f32": torch.float32, "bf16": torch.int16, "fp8": torch.uint8}[wl.dtype]


def np_elem(wl):
    """numpy dtype of the generator's raw K/V elements (bit patterns for bf16/fp8)."""
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[wl.dtype]


def index_torch_dtype(wl):
    """torch dtype of the Mean-K index (bf16 bits for bf16 and fp8 K)."""
    import torch
    return torch.float32 if wl.index_dtype == "f32" else torch.int16


def fp8_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of E4M3 values around |x| (subnormal step 2^-9)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


def to_dev(a: np.ndarray, dev):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host_bits(t) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.uint8:
        from oracle.numerics import fp8_decode
        return fp8_decode(a)
    return a.astype(np.float64)


def raw_to_device(wl, which: str, b0: int, nb: int, dev, chunk: int = 256):
    """Raw K or V of blocks [b0, b0+nb) as one device tensor [nb][block_elems]."""
    import torch
    out = torch.empty((nb, wl.block_elems), dtype=torch_dtype(wl), device=dev)
    for s in range(0, nb, chunk):
        n = min(chunk, nb - s)
        h = synth.kv_blocks(wl, which, b0 + s, n).reshape(n, -1)
        out[s:s + n].copy_(to_dev(h, "cpu"))
    return out


def build_index_dev(k, wl, raw_k, dev, cap: int | None = None, first: int = 0):
    import torch
    N = raw_k.shape[0]
    cap = cap or N
    index = torch.zeros((wl.n_layers, wl.n_kv_heads, cap, wl.head_dim),
                        dtype=index_torch_dtype(wl), device=dev)
    k.kvm_build_index(k.dims_for(wl), k.dtype_code(wl.dtype), raw_k, wl.block_bytes, first, N,
                      index, cap)
    return index


def score_dev(k, wl, q_dev, index, n_blocks: int, cap: int, dev, loc: int = 0,
              tile_blocks: int = 0, host_index=None):
    import torch
    dims = k.dims_for(wl)
    dt = k.dtype_code(wl.index_dtype)
    T = q_dev.shape[2]
    ws_b = k.kvm_score_ws_bytes(dims, dt, T, n_blocks, loc, tile_blocks)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    scores = torch.empty(n_blocks, dtype=torch.float32, device=dev)
    src = index if loc == 0 else host_index
    k.kvm_score_blocks(dims, dt, q_dev, T, src, cap, n_blocks, loc, tile_blocks, scores, ws, ws_b)
    return scores


def select_dev(k, scores, n_blocks: int, n_sink: int, n_recent: int, budget: int, dev, B: int = 32):
    import torch
    sel = torch.full((budget,), -7, dtype=torch.int32, device=dev)
    n_sel = torch.zeros(1, dtype=torch.int32, device=dev)
    base = torch.full((budget,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(k.kvm_select_ws_bytes(n_blocks), dtype=torch.uint8, device=dev)
    k.kvm_select(scores, n_blocks, n_sink, n_recent, budget, B, sel, n_sel, base, ws, ws.numel())
    return sel, n_sel, base


class Pool:
    """A page pool plus its context."""

    def __init__(self, k, wl, n_slots: int, max_blocks: int, max_pos: int, dev,
                 batch_blocks: int = 64, staging_blocks: int = 0, delta_limit: int = 0):
        import torch
        dt = torch_dtype(wl)
        self.k_view = torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev)
        self.v_view = torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev)
        # bounded delta re-RoPE keeps no raw-K shadow pages
        self.k_shadow = (None if delta_limit > 0 else
                         torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev))
        self.ctx = k.KvmCtx(k.dims_for(wl), k.dtype_code(wl.dtype), self.k_view, self.v_view,
                            self.k_shadow, n_slots, max_blocks, max_pos, wl.theta,
                            wl.rope_layout, batch_blocks, staging_blocks, delta_limit)
        self.page = torch.full((n_slots,), -1, dtype=torch.int32, device=dev)


def check_view(wl, sel: np.ndarray, page: np.ndarray, pool: Pool, blocks=None, atol=None):
    """Compare the K and V pages of selected blocks with the oracle.

    K: |K_gpu - RoPE(raw K)| within 2e-2 (bf16), half an E4M3 spacing plus
    the fp32 rotation's error (fp8) or 1e-5*max(1,|K|) (fp32), against the
    unrounded float64 oracle; V: bit-exact."""
    from oracle.pipeline import expected_view_k, expected_view_v_bits
    B = wl.block_tokens
    idx = range(len(sel)) if blocks is None else blocks
    worst = 0.0
    for i in idx:
        b = int(sel[i])
        slot = int(page[i])
        want = expected_view_k(wl, b, B * i)
        got = as_f64(to_host_bits(pool.k_view[slot])).reshape(want.shape)
        err = np.abs(got - want)
        if wl.dtype == "bf16":
            ok = np.all(err <= (atol if atol is not None else 2e-2))
        elif wl.dtype == "fp8":
            ok = np.all(err <= fp8_half_ulp(want * (1 + 1e-6)) + 1e-6 * np.maximum(1.0, np.abs(want)))
        else:
            ok = np.all(err <= 1e-5 * np.maximum(1.0, np.abs(want)))
        worst = max(worst, float(err.max()))
        assert ok, f"K of block {b} (view slot {i}) off by {err.max()}"
        vb = to_host_bits(pool.v_view[slot])
        assert np.array_equal(vb, expected_view_v_bits(wl, b).ravel()), f"V of block {b}"
    return worst


def build_index_streamed(k, wl, dev, n_blocks=None, chunk: int = 1024, cap=None):
    """Mean-K of blocks [0, n_blocks) built on the device from raw K that is
    generated on the host chunk by chunk (double-buffered pinned staging)."""
    import threading
    import torch
    N = n_blocks or wl.n_blocks
    cap = cap or N
    index = torch.zeros((wl.n_layers, wl.n_kv_heads, cap, wl.head_dim),
                        dtype=index_torch_dtype(wl), device=dev)
    stage = [torch.empty((chunk, wl.block_elems), dtype=torch_dtype(wl)).pin_memory()
             for _ in range(2)]
    dchunk = torch.empty((chunk, wl.block_elems), dtype=torch_dtype(wl), device=dev)
    starts = list(range(0, N, chunk))
    view = (lambda t: t.numpy().view(np.uint16)) if wl.dtype == "bf16" else (lambda t: t.numpy())

    def gen(i):
        s = starts[i]
        n = min(chunk, N - s)
        synth.kv_blocks(wl, "K", s, n, out=view(stage[i & 1])[:n])

    th = threading.Thread(target=gen, args=(0,))
    th.start()
    for i, s in enumerate(starts):
        th.join()
        n = min(chunk, N - s)
        dchunk[:n].copy_(stage[i & 1][:n])
        if i + 1 < len(starts):
            th = threading.Thread(target=gen, args=(i + 1,))
            th.start()
        k.kvm_build_index(k.dims_for(wl), k.dtype_code(wl.dtype), dchunk, wl.block_bytes, s, n,
                          index, cap)
        torch.cuda.synchronize()
    return index


def raw_blocks_to_device(wl, which: str, blocks, dev):
    """Raw K or V of an arbitrary list of blocks as one device tensor."""
    import torch
    h = torch.empty((len(blocks), wl.block_elems), dtype=torch_dtype(wl)).pin_memory()
    view = h.numpy().view(np.uint16) if wl.dtype == "bf16" else h.numpy()
    for i, b in enumerate(blocks):
        synth.kv_blocks(wl, which, int(b), 1, out=view[i:i + 1])
    return h.to(dev)


def check_selection(sel: np.ndarray, R_oracle: np.ndarray, n_sink: int, n_recent: int,
                    budget: int, band: float = 2e-5):
    """The GPU selection against the oracle's scores, deciding only what the
    scores decide: forced blocks present, the right count, ascending order,
    every candidate whose oracle score exceeds the cutoff score by more than
    `band` (relative) selected and every one below it by more than `band`
    left out. Candidates inside the band (fp32 vs fp64 rounding can order
    them either way) may go either way. Returns the number of band blocks."""
    N = len(R_oracle)
    sel = np.asarray(sel)
    assert np.all(np.diff(sel) > 0)
    if N <= budget:
        assert np.array_equal(sel, np.arange(N))
        return 0
    assert len(sel) == budget
    s = set(sel.tolist())
    assert set(range(n_sink)) <= s and set(range(N - n_recent, N)) <= s
    k = budget - n_sink - n_recent
    cand = np.arange(n_sink, N - n_recent)
    Rc = R_oracle[cand]
    cut = np.sort(Rc)[::-1][k - 1]
    above = cand[Rc > cut * (1 + band)]
    below = cand[Rc < cut * (1 - band)]
    assert set(above.tolist()) <= s, "a block clearly above the cutoff was not selected"
    assert not (set(below.tolist()) & s), "a block clearly below the cutoff was selected"
    return int(len(cand) - len(above) - len(below))


def pair_error_in_bound(got, exact, n_delta, layout):
    """Per (a, b) pair: |stored - exact| <= (n + 1) * sqrt(2)/2 ulp_bf16 of the
    pair's length (each store rounds, rotations keep earlier error's length),
    plus the fp32 rotation's own error. Returns the worst error in ulps."""
    if layout == 0:
        ea, eb = got[..., 0::2] - exact[..., 0::2], got[..., 1::2] - exact[..., 1::2]
        na, nb = exact[..., 0::2], exact[..., 1::2]
    else:
        h = got.shape[-1] // 2
        ea, eb = got[..., :h] - exact[..., :h], got[..., h:] - exact[..., h:]
        na, nb = exact[..., :h], exact[..., h:]
    err, norm = np.hypot(ea, eb), np.hypot(na, nb)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(1.1 * norm, 2.0 ** -100))) - 7)
    bound = (n_delta + 1) * (np.sqrt(2) / 2 * ulp + 1e-6 * norm)
    assert np.all(err <= bound)
    return float(np.max(err / (2.0 ** (np.floor(np.log2(np.maximum(norm, 2.0 ** -100))) - 7))))
