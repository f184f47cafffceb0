#!/usr/bin/env python3
"""One working-set update step on a seeded 1M-token workspace, on one MI355X.

Workspace: 32768 blocks of 32 tokens, 64 layers, 8 KV heads, 48 query heads,
head dim 128, bf16; 512 query tokens; budget 4096 blocks (sink 1, recent 64);
half of the selected blocks already resident in the page pool (prefilled,
K page stale), the other half staged from their lower-tier copy.

A timed step is the whole hot path: Mean-K append of the step's 16 freshly
prefilled blocks, scoring of all 32768 blocks (Eq. (10) of the KVMem paper),
selection, and rematerialization of the 4096-block view (2048 hits re-encoded
from their raw-K shadow pages, 2048 misses gathered + re-RoPE'd + V copied).
For `value` the misses' raw K/V sit in HBM; a second leg repeats the step
with the misses in pinned host memory (DMA on a side stream overlapped with
the scatter kernel) and is reported separately.

Prints one JSON line. See --help for options.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("history blocks scored/s + rematerialized KV GB/s (fraction of HBM peak), 1M-tok")
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# VALU issue bound of a score pass: per score element one fused scale-and-shift,
# one v_exp_f32 (half the fp32 issue rate, measured 1.4e13/s over the chip) and
# one add, i.e. 4 wave issue slots of 4 cycles per 64 elements on each of the
# 1024 SIMDs at 2.4 GHz: 1024 * 2.4e9 * 64 / 16 score elements per second.
VALU_SCORE_PEAK_GELEMS = 1024 * 2.4e9 * 64 / 16 / 1e9
MFMA_FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--pcie-steps", type=int, default=3,
                    help="steps of the pinned-host leg (0 to skip)")
    ap.add_argument("--delta-steps", type=int, default=4,
                    help="rematerializations timed in bounded delta re-RoPE mode (0: skip)")
    ap.add_argument("--fp8", type=int, default=1,
                    help="also time the view with FP8 E4M3 K/V pages (0: skip)")
    ap.add_argument("--median-runs", type=int, default=50,
                    help="runs of the kernel-median leg after 10 untimed ones (0: skip)")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="time the CPU oracle sample")
    ap.add_argument("--cpu-pairs", type=int, default=6,
                    help="(layer, KV head) pairs in the CPU oracle sample")
    ap.add_argument("--workload", default="ws1m", choices=["ws1m", "ctx64k", "churn", "ws10m"])
    ap.add_argument("--host-tiled", type=int, default=1,
                    help="10M-token workspace: also run the host-tiled legs (0: resident "
                         "legs only, as for its counter runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="first run a plain device copy of 2 GiB (counter calibration)")
    return ap.parse_args()


class Workspace:
    """Device-resident inputs and the page pool of one seeded workspace."""

    def __init__(self, k, wl, dev):
        import torch
        import synth
        self.k, self.wl, self.dev = k, wl, dev
        self.dims = k.dims_for(wl)
        self.dt = k.KVM_BF16
        N, nbytes = wl.n_blocks, wl.block_bytes
        self.N = N
        self.n_new = wl.n_q_tokens // wl.block_tokens          # blocks of this step's prefill
        self.index = torch.zeros((wl.n_layers, wl.n_kv_heads, N, wl.head_dim),
                                 dtype=torch.int16, device=dev)
        # --- Mean-K of the history, built from generated raw K in chunks ----
        chunk = 1024
        stage = [torch.empty((chunk, wl.block_elems), dtype=torch.int16).pin_memory()
                 for _ in range(2)]
        dchunk = torch.empty((chunk, wl.block_elems), dtype=torch.int16, device=dev)
        n_hist = N - self.n_new
        starts = list(range(0, n_hist, chunk))
        gen_err = []

        def gen(i):
            s = starts[i]
            n = min(chunk, n_hist - s)
            try:
                synth.kv_blocks(wl, "K", s, n, out=stage[i & 1].numpy()[:n].view(np.uint16))
            except Exception as e:  # pragma: no cover
                gen_err.append(e)

        t0 = time.time()
        th = threading.Thread(target=gen, args=(0,))
        th.start()
        # kernel-only durations from the library's own event pairs on its stream
        k.kvm_profile_enable(True)
        for i, s in enumerate(starts):
            th.join()
            if gen_err:
                raise gen_err[0]
            n = min(chunk, n_hist - s)
            dchunk[:n].copy_(stage[i & 1][:n], non_blocking=True)
            torch.cuda.current_stream().synchronize()
            if i + 1 < len(starts):
                th = threading.Thread(target=gen, args=(i + 1,))
                th.start()
            k.kvm_build_index(self.dims, self.dt, dchunk, nbytes, s, n, self.index, N)
            torch.cuda.current_stream().synchronize()
            if i % 16 == 0:
                log(f"index build {s + n}/{n_hist} blocks, {time.time() - t0:.1f}s")
        launches, ms = k.kvm_profile_read().get("build_index", (0, float("nan")))
        k.kvm_profile_enable(False)
        self.build_stats = {"launches": launches, "blocks": n_hist, "ms": ms}
        del dchunk, stage
        # this step's freshly prefilled blocks: raw K/V on the device
        self.new_k = self._gen_dev("K", n_hist, self.n_new)
        self.new_v = self._gen_dev("V", n_hist, self.n_new)
        k.kvm_build_index(self.dims, self.dt, self.new_k, nbytes, n_hist, self.n_new,
                          self.index, N)
        self.q = torch.from_numpy(synth.query(wl).view(np.int16)).to(dev)
        T = wl.n_q_tokens
        self.ws_bytes = k.kvm_score_ws_bytes(self.dims, self.dt, T, N)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.scores = torch.empty(N, dtype=torch.float32, device=dev)
        Kb = wl.budget_blocks
        self.sel = torch.empty(Kb, dtype=torch.int32, device=dev)
        self.n_sel = torch.empty(1, dtype=torch.int32, device=dev)
        self.base = torch.empty(Kb, dtype=torch.int32, device=dev)
        self.page = torch.empty(Kb, dtype=torch.int32, device=dev)
        self.sel_ws = torch.empty(k.kvm_select_ws_bytes(N), dtype=torch.uint8, device=dev)
        log(f"index ready in {time.time() - t0:.1f}s")

    def _gen_dev(self, which, b0, nb):
        import synth
        import torch
        h = torch.empty((nb, self.wl.block_elems), dtype=torch.int16).pin_memory()
        synth.kv_blocks(self.wl, which, b0, nb, out=h.numpy().view(np.uint16))
        return h.to(self.dev)

    def score_select(self):
        k, wl = self.k, self.wl
        k.kvm_score_blocks(self.dims, self.dt, self.q, wl.n_q_tokens, self.index, self.N, self.N,
                           k.KVM_INDEX_DEVICE, 0, self.scores, self.ws, self.ws_bytes)
        k.kvm_select(self.scores, self.N, wl.n_sink, wl.n_recent, wl.budget_blocks,
                     wl.block_tokens, self.sel, self.n_sel, self.base, self.sel_ws,
                     self.sel_ws.numel())

    def setup_pool(self, sel: np.ndarray):
        """Pool + context; even-ranked selected blocks resident, odd-ranked staged."""
        import synth
        import torch
        k, wl, dev = self.k, self.wl, self.dev
        self.hits = sel[0::2].copy()
        self.misses = sel[1::2].copy()
        n_slots = wl.budget_blocks + wl.append_blocks + 64
        dt = torch.int16
        self.k_view = torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev)
        self.v_view = torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev)
        self.k_shadow = torch.zeros((n_slots, wl.block_elems), dtype=dt, device=dev)
        max_pos = (wl.budget_blocks + wl.reserve_blocks) * wl.block_tokens
        self.ctx = k.KvmCtx(self.dims, self.dt, self.k_view, self.v_view, self.k_shadow, n_slots,
                            wl.final_blocks, max_pos, wl.theta, wl.rope_layout, 64)
        nh, nm = len(self.hits), len(self.misses)
        # raw K/V of the resident half (device; re-registered before every step)
        self.hit_k = torch.empty((nh, wl.block_elems), dtype=dt, device=dev)
        self.hit_v = torch.empty((nh, wl.block_elems), dtype=dt, device=dev)
        # lower-tier copies of the missing half: pinned host, and an HBM copy
        self.miss_k_h = torch.empty((nm, wl.block_elems), dtype=dt).pin_memory()
        self.miss_v_h = torch.empty((nm, wl.block_elems), dtype=dt).pin_memory()
        tmp = torch.empty((64, wl.block_elems), dtype=dt).pin_memory()
        tv = tmp.numpy().view(np.uint16)
        for which, dst in (("K", self.hit_k), ("V", self.hit_v)):
            for i, b in enumerate(self.hits):
                synth.kv_blocks(wl, which, int(b), 1, out=tv[i % 64:i % 64 + 1])
                if i % 64 == 63 or i == nh - 1:
                    s = i - (i % 64)
                    dst[s:i + 1].copy_(tmp[:i + 1 - s])
            torch.cuda.synchronize()
        for which, dst in (("K", self.miss_k_h), ("V", self.miss_v_h)):
            dv = dst.numpy().view(np.uint16)
            for i, b in enumerate(self.misses):
                synth.kv_blocks(wl, which, int(b), 1, out=dv[i:i + 1])
        self.miss_k_d = self.miss_k_h.to(dev)
        self.miss_v_d = self.miss_v_h.to(dev)
        torch.cuda.synchronize()

    def set_miss_sources(self, where: str):
        k, wl = self.k, self.wl
        kk, vv, loc = ((self.miss_k_d, self.miss_v_d, k.KVM_SRC_DEVICE) if where == "hbm" else
                       (self.miss_k_h, self.miss_v_h, k.KVM_SRC_HOST_PINNED))
        for i, b in enumerate(self.misses):
            self.ctx.kvm_ctx_set_source(int(b), 1, kk[i], vv[i], wl.block_bytes, loc)

    def reset_pool(self):
        """Back to the step's start: all pages free, then the resident half
        registered again as freshly prefilled (K page stale)."""
        wl = self.wl
        self.ctx.kvm_ctx_evict(0, wl.final_blocks)
        self.ctx.kvm_ctx_register_resident_list(self.hits, self.hit_k, self.hit_v,
                                                wl.block_bytes)

    def step(self):
        """The timed hot path of one agent step."""
        k, wl = self.k, self.wl
        k.kvm_build_index(self.dims, self.dt, self.new_k, wl.block_bytes, self.N - self.n_new,
                          self.n_new, self.index, self.N)
        self.score_select()
        return self.ctx.kvm_rematerialize(self.sel, self.n_sel, self.page)


def fp8_scores_leg(k, ws, wl, dev, steps: int, warmup: int) -> dict:
    """FP8 scoring ablation on the same workspace: the step's queries and the
    Mean-K index converted to E4M3 (kvm_quantize_e4m3), scored on the FP8
    matrix-core kernels and selected with the same budget; reports the pass
    times and how much of the bf16 selection's free part the FP8 one keeps."""
    import torch
    N, T = ws.N, wl.n_q_tokens
    q8 = torch.empty(ws.q.numel(), dtype=torch.uint8, device=dev)
    i8 = torch.empty(ws.index.numel(), dtype=torch.uint8, device=dev)
    k.kvm_quantize_e4m3(ws.q, k.KVM_BF16, ws.q.numel(), q8)
    k.kvm_quantize_e4m3(ws.index, k.KVM_BF16, ws.index.numel(), i8)
    wsb = k.kvm_score_ws_bytes(ws.dims, k.KVM_FP8_E4M3, T, N, 0, 0)
    sws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sc = torch.empty(N, dtype=torch.float32, device=dev)
    sel = torch.empty_like(ws.sel)
    n_sel = torch.empty_like(ws.n_sel)
    base = torch.empty_like(ws.base)

    def once():
        k.kvm_score_blocks(ws.dims, k.KVM_FP8_E4M3, q8, T, i8, N, N, k.KVM_INDEX_DEVICE, 0, sc,
                           sws, wsb)
        k.kvm_select(sc, N, wl.n_sink, wl.n_recent, wl.budget_blocks, wl.block_tokens, sel,
                     n_sel, base, ws.sel_ws, ws.sel_ws.numel())
    for _ in range(max(1, warmup)):
        once()
    torch.cuda.synchronize()
    k.kvm_profile_enable(True)
    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    prof = k.kvm_profile_read()
    k.kvm_profile_enable(False)
    kern = {n: c_t[1] / c_t[0] for n, c_t in prof.items()}
    ws.score_select()                          # the bf16 selection, for comparison
    torch.cuda.synchronize()
    n = int(ws.n_sel.item())
    a = set(ws.sel.cpu().numpy()[:n].tolist())
    b = set(sel.cpu().numpy()[:int(n_sel.item())].tolist())
    free = wl.budget_blocks - wl.n_sink - wl.n_recent
    flops = 2.0 * wl.n_layers * wl.n_q_heads * T * N * wl.head_dim
    p1, p2 = kern.get("score_pass1_mfma"), kern.get("score_pass2_mfma")
    out = {"pass1_ms": p1, "pass2_ms": p2,
           "score_ms": sum(v for n_, v in kern.items() if n_.startswith("score")),
           "pass1_TFLOPs": flops / (p1 * 1e-3) / 1e12 if p1 else None,
           "fp8_peak_TFLOPs": MFMA_FP8_PEAK_TFLOPS,
           "selection_kept_of_bf16_free": (len(a & b) - (n - free)) / free,
           "note": "E4M3 queries and Mean-K (round to nearest even, saturating); "
                   "fp32 accumulation, softmax as in bf16"}
    del q8, i8, sws
    log(f"fp8 scores: pass 1 {p1:.2f} ms, pass 2 {p2:.2f} ms, keeps "
        f"{100 * out['selection_kept_of_bf16_free']:.1f}% of the bf16 free selection")
    return out


def fp8_leg(k, ws, wl, dev, steps: int) -> dict:
    """The same view with FP8 E4M3 K/V pages (the KV format of the pages' engine):
    resident half registered, missing half from HBM copies, timed like the value
    leg; plus the Mean-K build from FP8 K over 1024 blocks."""
    import synth
    import torch
    w8 = synth.get_workload("ws1m_fp8")
    page = w8.block_bytes
    n_slots = ws.k_view.shape[0]
    pools = [torch.zeros((n_slots, w8.block_elems), dtype=torch.uint8, device=dev)
             for _ in range(3)]

    def blocks_to_dev(which, blocks):
        out = torch.empty((len(blocks), w8.block_elems), dtype=torch.uint8, device=dev)
        h = torch.empty((256, w8.block_elems), dtype=torch.uint8).pin_memory()
        hv = h.numpy()
        for s0 in range(0, len(blocks), 256):
            part = blocks[s0:s0 + 256]
            for i, b in enumerate(part):
                synth.kv_blocks(w8, which, int(b), 1, out=hv[i:i + 1])
            out[s0:s0 + len(part)].copy_(h[:len(part)])
        torch.cuda.synchronize()
        return out
    hk, hv_ = blocks_to_dev("K", ws.hits), blocks_to_dev("V", ws.hits)
    mk, mv = blocks_to_dev("K", ws.misses), blocks_to_dev("V", ws.misses)
    ctx = k.KvmCtx(ws.dims, k.KVM_FP8_E4M3, pools[0], pools[1], pools[2], n_slots,
                   wl.final_blocks, (wl.budget_blocks + wl.reserve_blocks) * wl.block_tokens,
                   wl.theta, wl.rope_layout, 64)
    for i, b in enumerate(ws.misses):
        ctx.kvm_ctx_set_source(int(b), 1, mk[i], mv[i], page, k.KVM_SRC_DEVICE)

    def one():
        ctx.kvm_ctx_evict(0, wl.final_blocks)
        ctx.kvm_ctx_register_resident_list(ws.hits, hk, hv_, page)
        torch.cuda.synchronize()
        return ctx.kvm_rematerialize(ws.sel, ws.n_sel, ws.page)
    one()
    torch.cuda.synchronize()
    k.kvm_profile_enable(True)
    for _ in range(steps):
        st = one()
    torch.cuda.synchronize()
    rc_, rt_ = k.kvm_profile_read().get("remat", (0, float("nan")))
    k.kvm_profile_enable(False)
    r_ms = rt_ / max(rc_, 1)
    r_bytes = st["hits"] * 2 * page + st["misses"] * 4 * page
    # Mean-K from FP8 K: 1024 blocks (the staged half's K copies)
    nb = min(1024, len(ws.misses))
    L, Hkv, d = w8.n_layers, w8.n_kv_heads, w8.head_dim
    idx = torch.empty((L, Hkv, nb, d), dtype=torch.int16, device=dev)
    k.kvm_build_index(ws.dims, k.KVM_FP8_E4M3, mk, page, 0, nb, idx, nb)
    torch.cuda.synchronize()
    k.kvm_profile_enable(True)
    for _ in range(3):
        k.kvm_build_index(ws.dims, k.KVM_FP8_E4M3, mk, page, 0, nb, idx, nb)
    torch.cuda.synchronize()
    bc, bt = k.kvm_profile_read().get("build_index", (0, float("nan")))
    k.kvm_profile_enable(False)
    b_ms = bt / max(bc, 1)
    b_bytes = nb * (page + L * Hkv * d * 2)
    ctx.close()
    del pools, hk, hv_, mk, mv, idx
    torch.cuda.empty_cache()
    out = {"page_bytes": page, "remat": {"avg_ms": r_ms, "bytes": r_bytes,
                                         "GBps": r_bytes / (r_ms * 1e-3) / 1e9,
                                         "hbm_frac": r_bytes / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                         "hits": st["hits"], "misses": st["misses"]},
           "build": {"blocks": nb, "avg_ms": b_ms, "GBps": b_bytes / (b_ms * 1e-3) / 1e9,
                     "hbm_frac": b_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}}
    log(f"fp8 leg: remat {r_ms:.2f} ms ({out['remat']['GBps']:.0f} GB/s), "
        f"Mean-K build {b_ms:.3f} ms ({out['build']['GBps']:.0f} GB/s)")
    return out


def measured_peaks(k, dev) -> dict:
    """Achievable rates on this GPU next to the datasheet peaks. The library's
    own measurement kernels (kvm_measure_rate: a STREAM-style copy of 2 GiB, a
    register-only bf16 MFMA loop, a v_exp_f32 loop and the score passes'
    MFMA + exp instruction mix at their occupancy, each about 50 ms after an
    untimed run) give the bounds the frac_of_measured fields use; vendor library
    calls (a 2 GiB torch copy, an 8192^3 torch.mm on the vendor BLAS, a 1 GiB
    copy from pinned host memory) are reported beside them."""
    import torch
    scratch = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    own = {"copy_kernel_GBps": k.kvm_measure_rate(k.KVM_RATE_COPY, 1 << 31, scratch) / 1e9,
           "mfma_loop_TFLOPs": k.kvm_measure_rate(k.KVM_RATE_MFMA_BF16, 200000, scratch) / 1e12,
           "exp_per_s": k.kvm_measure_rate(k.KVM_RATE_EXP, 200000, scratch),
           "score_mix_Gscores": k.kvm_measure_rate(k.KVM_RATE_SCORE_MIX, 400000, scratch) / 1e9}
    del scratch
    a = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    x = torch.randn(8192, 8192, device=dev).to(torch.bfloat16).contiguous()
    y = torch.randn(8192, 8192, device=dev).to(torch.bfloat16).contiguous()
    z = torch.empty_like(x)

    def rate(fn, reps):
        for _ in range(reps):       # bring the clocks up first: they ramp over tens of ms
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3
    t_copy = rate(lambda: b.copy_(a), 30)
    t_mm = rate(lambda: torch.mm(x, y, out=z), 40)
    h = torch.empty(1 << 30, dtype=torch.uint8).pin_memory()
    d = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    t_h2d = rate(lambda: d.copy_(h, non_blocking=True), 4)
    out = dict(own)
    out.update({"hbm_copy_GBps": 2 * a.numel() * 4 / t_copy / 1e9,
                "bf16_gemm_TFLOPs": 2 * 8192 ** 3 / t_mm / 1e12,
                "h2d_pinned_GBps": h.numel() / t_h2d / 1e9,
                "how": "own kernels (kvm_measure_rate): 2 GiB STREAM-style copy (bytes read + "
                       "written), bf16 MFMA loop, v_exp_f32 loop, and the score passes' "
                       "instruction mix (per MFMA two fma, two exp, two add; 2 waves per SIMD), "
                       "each one untimed and one timed run of about 50 ms; vendor calls: torch "
                       "copy_ of 2 GiB (30 untimed, 30 timed), torch.mm 8192^3 bf16 (40 untimed, "
                       "40 timed), a 1 GiB copy from pinned host memory (4 untimed, 4 timed)"})
    del a, b, x, y, z, h, d
    return out


def source_fingerprint(path: str) -> str:
    """First 16 hex digits of the SHA-256 of a source file with its comments and
    blank lines removed, so that only a change of code invalidates counters."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)      # block comments
    text = re.sub(r"//[^\n]*", "", text)                    # line comments
    code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def counter_traffic(name: str = "ws1m_traffic.json") -> dict:
    """HBM bytes per dispatch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (profiles/<name>), per kernel; a kernel whose source code (comments
    aside) changed since the counters were taken maps to None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    data = json.load(open(path))
    out = {}
    for name, v in data.get("per_dispatch", {}).items():
        src = os.path.join(ROOT, v["source"])
        ok = os.path.exists(src) and source_fingerprint(src) == v["source_sha256_16"]
        out[name] = (v["read_bytes"] + v["write_bytes"]) if ok else None
    return out


# Kernels whose counter traffic the bench line reports, as (name, template
# arguments): remat_kernel<element, head dim, pair layout, delta mode, V copy>
# for the view (full re-encodes and device misses) and for in-place shifts.
SCORE_KERNEL_TAIL = "<unsigned short, 128>"
REMAT_VIEW_KERNEL = ("remat_kernel", "<unsigned short, 128, 0, false, true>")
REMAT_DELTA_KERNEL = ("remat_kernel", "<unsigned short, 128, 0, true, false>")
# stored-score pass 1 of the 10M-token workspace: bf16, d = 128, LDS-staged stores
STORED_KERNEL_TAIL = "<unsigned short, 128, true>"


def traffic_for(traffic: dict, short: str, tail: str | None = None):
    for name, val in traffic.items():
        if name.split("<")[0].endswith(short) and (tail is None or name.endswith(tail)):
            return val
    return None


def workload_desc(wl) -> str:
    """The workload as the JSON line names it, from its own sizes."""
    label = {"ws1m": "1M-token workspace", "ctx64k": "64K-token history"}.get(
        wl.name, f"{wl.n_blocks * wl.block_tokens}-token workspace")
    return (f"{label}: {wl.n_blocks} blocks x {wl.block_tokens} tokens, {wl.n_layers} layers, "
            f"{wl.n_kv_heads} KV / {wl.n_q_heads} query heads, d {wl.head_dim}, "
            f"{wl.n_q_tokens} query tokens, budget {wl.budget_blocks} blocks (sink {wl.n_sink}, "
            f"recent {wl.n_recent}), half of the view resident in the page pool and the "
            f"other half's raw K/V read from a lower-tier copy in HBM (the same step with "
            f"that copy in pinned host memory, fetched over PCIe, is whole_step_host_tier)")


def kernel_medians(k, ws, runs: int, remat_bytes: int, warm: int = 10) -> dict:
    """Medians over `runs` launches of the score passes and the remat kernel,
    after `warm` untimed scorings: scorings back to back, each remat after the
    pool reset (outside its launch), every launch timed by the library's events."""
    import torch
    for _ in range(warm):
        ws.score_select()
    torch.cuda.synchronize()
    p1, p2, rm = [], [], []
    for _ in range(runs):
        k.kvm_profile_enable(True)
        ws.score_select()
        torch.cuda.synchronize()
        st = k.kvm_profile_read()
        k.kvm_profile_enable(False)
        p1.append(st["score_pass1_mfma"][1] / st["score_pass1_mfma"][0])
        p2.append(st["score_pass2_mfma"][1] / st["score_pass2_mfma"][0])
    calls = []
    for _ in range(runs):
        ws.reset_pool()
        torch.cuda.synchronize()
        k.kvm_profile_enable(True)
        t0 = time.perf_counter()
        ws.ctx.kvm_rematerialize(ws.sel, ws.n_sel, ws.page)
        torch.cuda.synchronize()
        calls.append(time.perf_counter() - t0)
        st = k.kvm_profile_read()
        k.kvm_profile_enable(False)
        rm.append(st["remat"][1])          # all remat launches of the call
    r = float(np.median(rm))
    c = float(np.median(calls)) * 1e3
    view = view_bytes(ws)
    # Mean-K build in steady state: one launch over the staged half's raw K,
    # already in HBM (2048 blocks, 8.25 GiB), after warm launches
    wl = ws.wl
    nb = ws.miss_k_d.shape[0]
    bidx = torch.empty((wl.n_layers, wl.n_kv_heads, nb, wl.head_dim), dtype=torch.int16,
                       device=ws.dev)
    bt = []
    for i in range(3 + max(5, runs // 5)):
        k.kvm_profile_enable(True)
        k.kvm_build_index(ws.dims, ws.dt, ws.miss_k_d, wl.block_bytes, 0, nb, bidx, nb)
        torch.cuda.synchronize()
        st = k.kvm_profile_read()
        k.kvm_profile_enable(False)
        if i >= 3:
            bt.append(st["build_index"][1])
    del bidx
    b_ms = float(np.median(bt))
    b_bytes = nb * (wl.block_bytes + wl.n_layers * wl.n_kv_heads * wl.head_dim * 2)
    return {"runs": runs, "warmup": warm, "score_pass1_ms": float(np.median(p1)),
            "build_blocks": nb, "build_ms": b_ms, "build_GBps": b_bytes / (b_ms * 1e-3) / 1e9,
            "build_hbm_frac": b_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "score_pass2_ms": float(np.median(p2)), "remat_ms": r,
            "remat_GBps": remat_bytes / (r * 1e-3) / 1e9,
            "remat_hbm_frac": remat_bytes / (r * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "remat_call_ms": c, "delivered_view_GBps": view / (c * 1e-3) / 1e9}


def view_bytes(ws) -> int:
    """K and V bytes of the execution view the rematerialization delivers."""
    return int(ws.n_sel.item()) * 2 * ws.wl.block_bytes


def timed_remat_call(k, ws, runs: int = 3) -> float:
    """Median wall time (s) of kvm_rematerialize from the pool's reset state, the
    selection already on the device: reading it back, planning, H2D, kernels."""
    import torch
    t = []
    for _ in range(runs):
        ws.reset_pool()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ws.ctx.kvm_rematerialize(ws.sel, ws.n_sel, ws.page)
        torch.cuda.synchronize()
        t.append(time.perf_counter() - t0)
    return float(np.median(t))


def cpu_baseline(wl, pairs: int) -> dict:
    """The oracle, as it stands, on a bounded sample of the same step."""
    import synth
    from oracle import pipeline as op
    from oracle.scores import lg_partial_scores
    from oracle.select import select_blocks
    from oracle.meank import mean_k
    from oracle.rope import rope_rotate
    try:
        from threadpoolctl import threadpool_info
        cores = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    N, d = wl.n_blocks, wl.head_dim
    G, T = wl.group, wl.n_q_tokens
    rng = np.random.default_rng(0)
    # scoring: `pairs` (layer, KV head) pairs over all N blocks (index drawn
    # directly, same shape; the oracle's cost does not depend on the values)
    sub = wl.scaled(n_layers=1)
    idx = op.as_f64(synth.index_direct(sub, 0, N), "bf16")          # [1][Hkv][N][d]
    q = op.as_f64(synth.query(sub), "bf16")                          # [1][Hq][T][d]
    t0 = time.perf_counter()
    for p in range(pairs):
        lg_partial_scores(q, idx, 0, p % wl.n_kv_heads)
    t_pair = (time.perf_counter() - t0) / pairs
    # Mean-K of the step's new blocks (16 of them), selection, re-RoPE of 8 blocks
    t0 = time.perf_counter()
    nb = 2
    mean_k(op.raw_blocks(wl, "K", 0, nb), "bf16")
    t_mk = (time.perf_counter() - t0) / nb
    R = rng.random(N)
    t0 = time.perf_counter()
    select_blocks(R, wl.n_sink, wl.n_recent, wl.budget_blocks)
    t_sel = time.perf_counter() - t0
    t0 = time.perf_counter()
    nr = 4
    for i in range(nr):
        kb = op.raw_blocks(wl, "K", i, 1)[0]
        rope_rotate(kb, 32 * i + np.arange(32), wl.theta, wl.rope_layout)
    t_rope = (time.perf_counter() - t0) / nr
    n_pairs = wl.n_layers * wl.n_kv_heads
    est = t_pair * n_pairs + t_mk * (T // 32) + t_sel + t_rope * wl.budget_blocks
    return {"value": N / est, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float64 NumPy oracle: Eq. (10) partial scores of {pairs} of "
                       f"{n_pairs} (layer, KV head) pairs over all {N} blocks "
                       f"({t_pair:.2f} s each), Mean-K of {nb} blocks, one selection, "
                       f"re-RoPE of {nr} blocks; extrapolated to one full step "
                       f"({est:.0f} s)"),
            "est_step_s": est}


def index_from_generated_k(k, upd, wl, dev, n_blocks: int, chunk: int = 1024):
    """Mean-K of the history built with the library from raw K generated on the
    host in chunks (double-buffered pinned staging); returns build stats."""
    import torch
    import synth
    stage = [torch.empty((chunk, wl.block_elems), dtype=torch.int16).pin_memory()
             for _ in range(2)]
    dchunk = torch.empty((chunk, wl.block_elems), dtype=torch.int16, device=dev)
    starts = list(range(0, n_blocks, chunk))

    def gen(i):
        s0 = starts[i]
        synth.kv_blocks(wl, "K", s0, min(chunk, n_blocks - s0),
                        out=stage[i & 1].numpy()[:min(chunk, n_blocks - s0)].view(np.uint16))

    th = threading.Thread(target=gen, args=(0,))
    th.start()
    t0 = time.time()
    for i, s0 in enumerate(starts):
        th.join()
        n = min(chunk, n_blocks - s0)
        dchunk[:n].copy_(stage[i & 1][:n])
        if i + 1 < len(starts):
            th = threading.Thread(target=gen, args=(i + 1,))
            th.start()
        upd.build(dchunk, s0, n)
        torch.cuda.synchronize()
        if i % 8 == 0:
            log(f"index build {s0 + n}/{n_blocks} blocks, {time.time() - t0:.1f}s")


def run_ws10m(args, k, wl, dev):
    """The 10M-token workspace (decode-style single query token): scoring of all
    312500 blocks and selection, with the directly drawn 41 GB index resident in
    HBM, and streamed from pinned host memory in 64 MiB tiles (the pages'
    host-resident index). Scoring and selection only: no page pool here."""
    import torch
    import synth
    N, tb, d = wl.n_blocks, wl.tile_blocks, wl.head_dim
    L, Hkv, Hq = wl.n_layers, wl.n_kv_heads, wl.n_q_heads
    nlg = L * Hkv
    ntile = (N + tb - 1) // tb
    t0 = time.time()
    host = torch.empty((ntile, nlg, tb, d), dtype=torch.int16).pin_memory()
    hv = host.numpy().view(np.uint16)
    for t in range(ntile):
        synth.index_direct(wl, t * tb, min(tb, N - t * tb), out=hv[t], lg_stride_elems=tb * d)
        if t % 100 == 0:
            log(f"index tiles {t}/{ntile}, {time.time() - t0:.1f}s")
    index = torch.empty((L, Hkv, N, d), dtype=torch.int16, device=dev)
    iv = index.view(nlg, N, d)
    for t in range(ntile):
        nb = min(tb, N - t * tb)
        iv[:, t * tb:t * tb + nb, :].copy_(host[t, :, :nb, :].to(dev))
    q = torch.from_numpy(synth.query(wl).view(np.int16)).to(dev)
    dims, bf = k.dims_for(wl), k.KVM_BF16
    scores = torch.empty(N, dtype=torch.float32, device=dev)
    sel = torch.empty(wl.budget_blocks, dtype=torch.int32, device=dev)
    n_sel = torch.empty(1, dtype=torch.int32, device=dev)
    base = torch.empty(wl.budget_blocks, dtype=torch.int32, device=dev)
    sel_ws = torch.empty(k.kvm_select_ws_bytes(N), dtype=torch.uint8, device=dev)
    log(f"setup {time.time() - t0:.1f}s")

    def leg(loc, dt=bf, qq=q, dev_index=index, host_index=host):
        wsb = k.kvm_score_ws_bytes(dims, dt, 1, N, loc, tb if loc else 0)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        src, tiles = (dev_index, 0) if loc == k.KVM_INDEX_DEVICE else (host_index, tb)

        def step():
            k.kvm_score_blocks(dims, dt, qq, 1, src, N, N, loc, tiles, scores, ws, wsb)
            k.kvm_select(scores, N, wl.n_sink, wl.n_recent, wl.budget_blocks, wl.block_tokens,
                         sel, n_sel, base, sel_ws, sel_ws.numel())
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        k.kvm_profile_enable(True)
        t1 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t1) * 1e3 / args.steps
        prof = k.kvm_profile_read()
        k.kvm_profile_enable(False)
        out = scores.clone()
        del ws
        return ms, {n: {"launches": c, "avg_ms": t / c} for n, (c, t) in prof.items()}, out
    tiled = bool(args.host_tiled)
    ms_res, kern_res, r_res = leg(k.KVM_INDEX_DEVICE)
    if tiled:
        ms_til, kern_til, r_til = leg(k.KVM_INDEX_HOST_TILED)
        assert torch.equal(r_res, r_til), "resident and host-tiled scores differ"
    # FP8 scoring ablation: the same index and query encoded to E4M3 on the GPU;
    # the host tiles reuse the pinned buffer (tile-major, 1 byte per element)
    i8 = torch.empty((nlg, N, d), dtype=torch.uint8, device=dev)
    q8 = torch.empty(q.numel(), dtype=torch.uint8, device=dev)
    k.kvm_quantize_e4m3(index, bf, index.numel(), i8)
    k.kvm_quantize_e4m3(q, bf, q.numel(), q8)
    h8 = host.view(-1).view(torch.uint8)[:ntile * nlg * tb * d].view(ntile, nlg, tb, d)
    for t in range(ntile):
        nb = min(tb, N - t * tb)
        h8[t, :, :nb, :].copy_(i8[:, t * tb:t * tb + nb, :].cpu())
    ms_f8, kern_f8, r_f8 = leg(k.KVM_INDEX_DEVICE, k.KVM_FP8_E4M3, q8, i8, h8)
    if tiled:
        ms_f8t, kern_f8t, r_f8t = leg(k.KVM_INDEX_HOST_TILED, k.KVM_FP8_E4M3, q8, i8, h8)
        assert torch.equal(r_f8, r_f8t), "resident and host-tiled FP8 scores differ"
    f8_rel = float(((r_f8.double() - r_res.double()).abs() / r_res.double()).max())
    idx_bytes = N * nlg * d * 2
    s_bytes = 2 * N * L * Hq * 4            # stored scores written and read back
    p1 = kern_res.get("score_stored_pass1", {}).get("avg_ms")
    p2 = kern_res.get("score_stored_pass2", {}).get("avg_ms")
    res = {"ms_per_step": ms_res, "blocks_per_s": N / (ms_res * 1e-3),
           "pass1_GBps": (idx_bytes + s_bytes / 2) / (p1 * 1e-3) / 1e9 if p1 else None,
           "pass2_GBps": (s_bytes / 2) / (p2 * 1e-3) / 1e9 if p2 else None,
           "kernels": kern_res}
    til = {"ms_per_step": ms_til, "blocks_per_s": N / (ms_til * 1e-3),
           "h2d_GBps": idx_bytes / (ms_til * 1e-3) / 1e9, "tile_bytes": nlg * tb * d * 2,
           "kernels": kern_til} if tiled else None
    f8p1 = kern_f8.get("score_stored_pass1", {}).get("avg_ms")
    fp8 = {"resident": {"ms_per_step": ms_f8, "blocks_per_s": N / (ms_f8 * 1e-3),
                        "pass1_GBps": (idx_bytes / 2 + s_bytes / 2) / (f8p1 * 1e-3) / 1e9
                        if f8p1 else None, "kernels": kern_f8},
           "host_tiled": {"ms_per_step": ms_f8t, "blocks_per_s": N / (ms_f8t * 1e-3),
                          "h2d_GBps": idx_bytes / 2 / (ms_f8t * 1e-3) / 1e9,
                          "tile_bytes": nlg * tb * d, "kernels": kern_f8t} if tiled else None,
           "max_rel_diff_vs_bf16": f8_rel}
    # the dominant kernel, stored-score pass 1, is HBM-bound: the index read once
    # plus the stored scores written
    scratch = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    copy_gbps = k.kvm_measure_rate(k.KVM_RATE_COPY, 1 << 31, scratch) / 1e9
    del scratch
    roof = None
    if p1:
        ach = res["pass1_GBps"]
        traffic = counter_traffic("ws10m_traffic.json")
        roof = {"kernel": "score_stored_pass1", "bound": "hbm", "achieved": ach,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                "traffic": traffic_for(traffic, "score_stored_pass1_mfma", STORED_KERNEL_TAIL),
                "frac_of_measured": ach / copy_gbps}
    log(f"resident: {ms_res:.2f} ms/step; FP8 resident {ms_f8:.2f} ms/step" +
        (f"; host-tiled: {ms_til:.1f} ms/step ({til['h2d_GBps']:.1f} GB/s of index over "
         f"PCIe); FP8 host-tiled {ms_f8t:.1f} ms/step" if tiled else ""))
    print(json.dumps({
        "metric": "history blocks scored/s, 10M-token workspace", "value": N / (ms_res * 1e-3),
        "unit": "blocks/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_res, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (directly drawn Mean-K index; seeded counter-based generator)",
        "config": {"workload": "10M-token workspace: 312500 blocks, 64 layers, 8 KV / 48 query "
                               "heads, d 128, 1 query token, budget 2048 blocks (sink 1, "
                               "recent 256); scoring + selection",
                   "tile_blocks": tb},
        "roofline": roof, "peaks_measured": {"copy_kernel_GBps": copy_gbps},
        "resident": res, "host_tiled": til, "fp8_scores": fp8,
    }), flush=True)


def run_churn(args, k, wl, dev):
    """The step-churn workspace: every step appends 64 freshly prefilled blocks
    and updates the working set; resident pages are reused, misses are gathered
    from a generator-backed lower tier through the pinned staging ring."""
    import torch
    import synth
    steps = min(args.steps, wl.steps)
    Kb, B = wl.budget_blocks, wl.block_tokens
    upd = k.WorkingSetUpdater(k.dims_for(wl), k.KVM_BF16, wl.final_blocks, Kb, wl.n_sink,
                              wl.n_recent, Kb + wl.append_blocks + 64,
                              (Kb + wl.reserve_blocks) * B, dev, wl.theta, wl.rope_layout,
                              batch_blocks=64, staging_blocks=256)
    index_from_generated_k(k, upd, wl, dev, wl.n_blocks)
    fn, user, keep = synth.gather_store(wl)
    upd.ctx.kvm_ctx_set_gather_raw(0, wl.final_blocks, fn, user)
    new_k = torch.empty((wl.append_blocks, wl.block_elems), dtype=torch.int16, device=dev)
    new_v = torch.empty_like(new_k)
    rows, prev = [], None
    trace = []                  # (new, selection, GPU misses) per step, for the host-tier replay
    k.kvm_profile_enable(True)
    for t in range(steps):
        q = torch.from_numpy(synth.query(wl, step=t).view(np.int16)).to(dev)
        if t > 0:
            b0 = upd.n_blocks
            new_k.copy_(torch.from_numpy(synth.kv_blocks(wl, "K", b0, wl.append_blocks).view(
                np.int16).reshape(wl.append_blocks, -1)))
            new_v.copy_(torch.from_numpy(synth.kv_blocks(wl, "V", b0, wl.append_blocks).view(
                np.int16).reshape(wl.append_blocks, -1)))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        new_ids = []
        if t > 0:
            new_ids = list(range(upd.n_blocks, upd.n_blocks + wl.append_blocks))
            upd.append(new_k, new_v, wl.append_blocks)
        upd.score(q, wl.n_q_tokens)
        upd.select()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        n = int(upd.n_sel.item())
        sel = upd.sel.cpu().numpy()[:n]
        # outside the timed region: which selected blocks the GPU pool lacks
        miss_ids = [int(b) for b in sel if upd.ctx.kvm_ctx_block_state(int(b))[0] < 0]
        trace.append((new_ids, sel.tolist(), miss_ids))
        t0 = time.perf_counter()
        st = upd.rematerialize()
        torch.cuda.synchronize()
        dt += time.perf_counter() - t0
        assert st["misses"] == len(miss_ids)
        cand = set(sel[(sel >= wl.n_sink) & (sel < upd.n_blocks - wl.n_recent)].tolist())
        ov = None if prev is None else len(cand & prev) / max(1, len(cand))
        prev = cand
        rows.append({"step": t, "ms": dt * 1e3, "n_blocks": upd.n_blocks, "overlap": ov, **st})
        log(f"churn step {t}: {dt * 1e3:.1f} ms, hits {st['hits']}, misses {st['misses']}, "
            f"evicted {st['evicted']}, overlap {ov}")
    prof = k.kvm_profile_read()
    k.kvm_profile_enable(False)
    upd.close()
    # Host-tier admission on the recorded trace (KVMem Sec. 4.4): NVMe reads of the
    # GPU misses for host tiers of 1x, 2x and 4x the view, LRU vs LRFU
    tier = []
    for cap in (Kb, 2 * Kb, 4 * Kb):
        for name, code, lam in (("lru", k.KVM_TIER_LRU, 0.0), ("lrfu", k.KVM_TIER_LRFU, 0.02),
                                ("lrfu", k.KVM_TIER_LRFU, 0.1), ("lrfu", k.KVM_TIER_LRFU, 0.5)):
            t1 = time.perf_counter()
            res = k.kvm_tier_simulate(code, cap, lam, trace)
            sim_ms = (time.perf_counter() - t1) * 1e3
            tier.append({"host_blocks": cap, "policy": name, "lambda": lam,
                         "host_hits": sum(r[0] for r in res), "nvme_reads": sum(r[1] for r in res),
                         "demotions": sum(r[2] for r in res), "sim_ms": sim_ms})
            log(f"host tier {cap} blocks, {name} {lam}: NVMe reads {tier[-1]['nvme_reads']}, "
                f"host hits {tier[-1]['host_hits']}")
    later = rows[1:] if len(rows) > 1 else rows
    ms = sum(r["ms"] for r in later) / len(later)
    ovs = [r["overlap"] for r in rows if r["overlap"] is not None]
    out = {
        "metric": METRIC, "value": wl.final_blocks / (ms * 1e-3), "unit": "blocks/s",
        "n_gpus": 1, "steps": steps, "warmup": 0, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": "step churn: 1M-token workspace, +64 blocks per step, "
                               "lower tier regenerated on demand by host gather workers",
                   "steps": steps},
        "mean_overlap": sum(ovs) / len(ovs) if ovs else None,
        "mean_hits": sum(r["hits"] for r in later) / len(later),
        "mean_misses": sum(r["misses"] for r in later) / len(later),
        "host_tier": tier,
        "steps_detail": rows,
        "kernels": {n: {"launches": c, "avg_ms": t / c} for n, (c, t) in prof.items()},
    }
    print(json.dumps(out), flush=True)



# ---------------------------------------------------------------------------
# rocprofv3 summaries (the profiles/ files are written from these)

def _short_kernel(n: str) -> str:
    return n.replace("void ", "").split("(")[0]


def summarize_rocprof(d: str) -> dict:
    """Per-kernel durations of <d>/kt and calibrated HBM bytes per dispatch from
    the FETCH_SIZE (<d>/pmc_fetch) and WRITE_SIZE (<d>/pmc_write) runs, scaled by
    what the same counters read for the 2 GiB elementwise copy that
    --calibrate-copy launches; written to <d>/summary.json."""
    import collections
    import glob
    import sqlite3

    def db(sub):
        f = sorted(glob.glob(os.path.join(d, sub, "*_results.db")))
        return f[0] if f else None
    out = {"kernels": {}, "calibration": {}, "traffic": {}}
    if db("kt"):
        con = sqlite3.connect(db("kt"))
        for n, c, tot, avg, pct in con.execute(
                "select name,total_calls,total_duration,average,percentage from top_kernels"):
            out["kernels"][_short_kernel(n)] = {"calls": c, "total_ms": tot / 1e3, "avg_us": avg,
                                               "pct": pct}

    def pmc(path, cname):
        agg = collections.defaultdict(list)
        if path:
            con = sqlite3.connect(path)
            for n, c, v in con.execute(
                    "select kernel_name, counter_name, value from counters_collection"):
                if c == cname:
                    agg[_short_kernel(n)].append(v)
        return {k: sum(v) / len(v) for k, v in agg.items()}
    f = pmc(db("pmc_fetch"), "FETCH_SIZE")
    w = pmc(db("pmc_write"), "WRITE_SIZE")
    # the 2 GiB copy of --calibrate-copy: torch.add(a, 0.0, out=b) on fp32
    cal = [k for k in set(f) | set(w) if "elementwise" in k and "OnSelf_add<float>" in k]
    if cal:
        c = cal[0]
        known = 2 * 1024 * 1024                   # KiB read and KiB written by the copy
        ff = known / f[c] if f.get(c) else None
        wf = known / w[c] if w.get(c) else None
        out["calibration"] = {"copy_kernel": c, "known_read_kib": known, "fetch_kib": f.get(c),
                              "write_kib": w.get(c), "fetch_factor": ff, "write_factor": wf}
        for k in sorted(set(f) | set(w)):
            if k.startswith("kvm::"):
                out["traffic"][k] = {
                    "fetch_kib_raw": f.get(k), "write_kib_raw": w.get(k),
                    "read_bytes": f.get(k, 0) * 1024 * ff if ff else None,
                    "write_bytes": w.get(k, 0) * 1024 * wf if wf else None}
    json.dump(out, open(os.path.join(d, "summary.json"), "w"), indent=1)
    return out


# the library's kernels by name prefix (after "kvm::") and the file each is defined in
KERNEL_SOURCES = {"score_": "attention_space_block_amd/csrc/score.hip",
                  "remat_kernel": "attention_space_block_amd/csrc/remat.hip",
                  "register_copy_kernel": "attention_space_block_amd/csrc/remat.hip",
                  "build_index": "attention_space_block_amd/csrc/build_index.hip",
                  "quantize_": "attention_space_block_amd/csrc/quantize.hip",
                  "sel_": "attention_space_block_amd/csrc/select.hip",
                  "select_": "attention_space_block_amd/csrc/select.hip",
                  "probe_": "attention_space_block_amd/csrc/probe.hip"}


def _source_of(kernel: str) -> str | None:
    """Source file of a library kernel (None for kernels the library does not
    define, e.g. the calibration copy)."""
    if not kernel.startswith("kvm::"):
        return None
    name = kernel[len("kvm::"):]
    for prefix, path in KERNEL_SOURCES.items():
        if name.startswith(prefix):
            return path
    return None


def write_traffic_profile(value_dir: str, delta_dir: str, out_path: str) -> dict:
    """profiles/ws1m_traffic.json: calibrated read/write bytes per dispatch of
    the value leg's kernels plus the delta-mode remat kernel of the delta leg,
    each with the fingerprint of its source (bench.py drops a kernel's traffic
    once its code changes)."""
    v = json.load(open(os.path.join(value_dir, "summary.json")))
    dl = json.load(open(os.path.join(delta_dir, "summary.json")))
    traffic = dict(v["traffic"])
    for k, x in dl["traffic"].items():
        # the delta-mode remat kernel: remat_kernel<T, D, LAYOUT, DELTA = true, COPYV>
        args = k.split("<", 1)[-1].rstrip(">").split(", ")
        if k.startswith("kvm::remat_kernel") and len(args) > 3 and args[3] == "true":
            traffic[k] = x
    per = {}
    for k, x in traffic.items():
        src = _source_of(k)
        if src:
            per[k] = dict(x, source=src,
                          source_sha256_16=source_fingerprint(os.path.join(ROOT, src)))
    out = {"workload": "1M-token workspace step (bench.py defaults; the delta-mode kernel from "
                       "the delta leg)", "calibration": v["calibration"], "per_dispatch": per}
    json.dump(out, open(out_path, "w"), indent=1)
    return out

# workloads with a traffic file of their own: profiles/<name>_traffic.json
# written from one counter run by --write-traffic-run <dir> <name>
TRAFFIC_RUNS = {"ws10m": "10M-token workspace, resident index legs (bench.py --workload ws10m "
                         "--host-tiled 0)",
                "ctx64k": "64K-token history step (bench.py --workload ctx64k)"}


def write_traffic_profile_run(run_dir: str, name: str) -> dict:
    """profiles/<name>_traffic.json: calibrated read/write bytes per dispatch of
    one workload's counter run, with source fingerprints as above."""
    v = json.load(open(os.path.join(run_dir, "summary.json")))
    per = {}
    for k, x in v["traffic"].items():
        src = _source_of(k)
        if src:
            per[k] = dict(x, source=src,
                          source_sha256_16=source_fingerprint(os.path.join(ROOT, src)))
    out = {"workload": TRAFFIC_RUNS[name], "calibration": v["calibration"], "per_dispatch": per}
    json.dump(out, open(os.path.join(ROOT, "profiles", f"{name}_traffic.json"), "w"), indent=1)
    return out


def main():
    if len(sys.argv) > 3 and sys.argv[1] == "--write-traffic-run":
        write_traffic_profile_run(sys.argv[2], sys.argv[3])
        return
    if len(sys.argv) > 2 and sys.argv[1] == "--summarize-rocprof":
        print(json.dumps(summarize_rocprof(sys.argv[2])["calibration"]))
        return
    if len(sys.argv) > 4 and sys.argv[1] == "--write-traffic":
        write_traffic_profile(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; pass --gpus 1"}))
        sys.exit(2)
    import torch
    import attention_space_block_amd as k
    import synth
    k._abi.lib()
    wl = synth.get_workload(args.workload)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        # a plain elementwise copy of known size: 2 GiB read + 2 GiB written
        a = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()
        del a, b
    if args.workload == "churn":
        run_churn(args, k, wl, dev)
        return
    if args.workload == "ws10m":
        run_ws10m(args, k, wl, dev)
        return
    t_setup = time.time()
    ws = Workspace(k, wl, dev)
    ws.score_select()
    torch.cuda.synchronize()
    n = int(ws.n_sel.item())
    sel0 = ws.sel.cpu().numpy()[:n]
    ws.setup_pool(sel0)
    ws.set_miss_sources("hbm")
    log(f"setup done in {time.time() - t_setup:.1f}s; view {n} blocks, "
        f"{len(ws.hits)} resident, {len(ws.misses)} staged")

    def run(n_steps, profile):
        times, stats = [], None
        for _ in range(n_steps):
            k.kvm_profile_enable(False)       # the reset is not part of the step
            ws.reset_pool()
            torch.cuda.synchronize()
            if profile:
                k.kvm_profile_enable(True)    # keeps the earlier steps' launches
            t0 = time.perf_counter()
            stats = ws.step()
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        return times, stats

    run(args.warmup, False)
    times, stats = run(args.steps, True)
    prof = k.kvm_profile_read()
    k.kvm_profile_enable(False)
    ms = 1e3 * sum(times) / len(times)
    sel_now = ws.sel.cpu().numpy()[:n]
    assert np.array_equal(sel_now, sel0), "selection changed between steps"
    log(f"value leg: {ms:.2f} ms/step, stats {stats}")
    kern = {name: {"launches": c, "avg_ms": t / c} for name, (c, t) in prof.items()}
    L, Hq, T, N, d = wl.n_layers, wl.n_q_heads, wl.n_q_tokens, wl.n_blocks, wl.head_dim
    flops_pass = 2.0 * L * Hq * T * N * d
    page = wl.block_bytes
    nh, nm = len(ws.hits), len(ws.misses)
    remat_bytes = nh * 2 * page + nm * 4 * page
    remat = kern.get("remat")
    if remat:
        # kernel time of one step's rematerialization (all its remat launches)
        remat["per_step_ms"] = remat["avg_ms"] * remat["launches"] / args.steps
    remat_gbps = remat_bytes / (remat["per_step_ms"] * 1e-3) / 1e9 if remat else None
    # rooflines: the dominant kernel of the step, and the other kernels of the path;
    # each workload reads the counters taken on its own runs (none: null traffic)
    traffic = (counter_traffic() if args.workload == "ws1m" else
               counter_traffic(f"{args.workload}_traffic.json"))

    def roofline(name, info):
        if name.startswith("score_pass"):
            ach = flops_pass / (info["avg_ms"] * 1e-3) / 1e12
            return {"kernel": name, "bound": "mfma", "achieved": ach,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic_for(traffic, name, SCORE_KERNEL_TAIL)}
        if name == "remat":
            return {"kernel": name, "bound": "hbm", "achieved": remat_gbps,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": remat_gbps / HBM_PEAK_GBPS,
                    "traffic": traffic_for(traffic, *REMAT_VIEW_KERNEL)}
        return None

    dom = max(kern.items(), key=lambda kv: kv[1]["avg_ms"] * kv[1]["launches"])
    roof = roofline(*dom)
    others = [roofline(n, i) for n, i in kern.items() if n != dom[0] and roofline(n, i)]
    # the score passes against their VALU issue bound (exps and sums of every score)
    elems = float(L * Hq * T * N)
    for n_ in ("score_pass1_mfma", "score_pass2_mfma"):
        if n_ in kern:
            ach = elems / (kern[n_]["avg_ms"] * 1e-3) / 1e9
            others.append({"kernel": n_, "bound": "alu", "achieved": ach,
                           "peak": VALU_SCORE_PEAK_GELEMS, "unit": "Gscores/s",
                           "frac": ach / VALU_SCORE_PEAK_GELEMS, "traffic": None})
    # PCIe leg: misses from pinned host memory. It runs right after the value
    # leg: run after the other legs and the peak measurements, its remat call
    # fell into a mode with about 35 GB/s of H2D in most processes (fast again
    # in a fresh process, and never in this order)
    pcie = None
    if args.pcie_steps > 0:
        ws.set_miss_sources("pinned")
        run(1, False)          # untimed: the first DMA from the pinned store pays one-time costs
        ptimes, pst = run(args.pcie_steps, False)
        pms = 1e3 * sum(ptimes) / len(ptimes)
        log("pcie leg steps (ms): " + ", ".join(f"{1e3 * t:.1f}" for t in ptimes))
        rc_s = timed_remat_call(k, ws)
        pcie = {"ms_per_step": pms, "blocks_per_s": N / (pms * 1e-3),
                "step_ms": [1e3 * t for t in ptimes],
                "remat_call_ms": rc_s * 1e3,
                "delivered_view_GBps": view_bytes(ws) / rc_s / 1e9,
                "h2d_bytes": pst["h2d_bytes"], "batches": pst["batches"],
                "step_h2d_GBps": pst["h2d_bytes"] / (pms * 1e-3) / 1e9,
                "frac_of_h2d_peak_measured": None}
        log(f"pcie leg: {pms:.2f} ms/step")
        ws.set_miss_sources("hbm")
    peaks = measured_peaks(k, dev)
    if pcie:
        pcie["frac_of_h2d_peak_measured"] = pcie["step_h2d_GBps"] / peaks["h2d_pinned_GBps"]
    measured_bound = {"mfma": peaks["mfma_loop_TFLOPs"], "hbm": peaks["copy_kernel_GBps"],
                      "alu": peaks["score_mix_Gscores"]}
    for r in [roof] + others:
        if r is not None and r["bound"] in measured_bound:
            r["frac_of_measured"] = r["achieved"] / measured_bound[r["bound"]]
    log(f"measured peaks: {peaks['copy_kernel_GBps']:.0f} GB/s own copy, "
        f"{peaks['mfma_loop_TFLOPs']:.0f} TFLOP/s MFMA loop, {peaks['exp_per_s']:.3g} exp/s, "
        f"{peaks['score_mix_Gscores']:.0f} G scores/s score mix; vendor: "
        f"{peaks['hbm_copy_GBps']:.0f} GB/s copy, {peaks['bf16_gemm_TFLOPs']:.0f} TFLOP/s GEMM")
    bst = ws.build_stats
    build_bytes = bst["blocks"] * (page + L * wl.n_kv_heads * d * 2)
    build_gbps = build_bytes / (bst["ms"] * 1e-3) / 1e9
    # Mean-K from K that carries RoPE (the prefill-time form), over 1024 blocks of
    # HBM-resident K (the staged half's copies stand in for cached K)
    nr = min(1024, nm)
    ridx = torch.empty((L, wl.n_kv_heads, nr, d), dtype=torch.int16, device=dev)
    ws.ctx.kvm_ctx_build_index_rope(ws.miss_k_d, page, 0, nr, 0, ridx, nr)
    torch.cuda.synchronize()
    k.kvm_profile_enable(True)
    for _ in range(3):
        ws.ctx.kvm_ctx_build_index_rope(ws.miss_k_d, page, 0, nr, 0, ridx, nr)
    torch.cuda.synchronize()
    rc_, rt_ = k.kvm_profile_read().get("build_index_rope", (0, float("nan")))
    k.kvm_profile_enable(False)
    del ridx
    rope_ms = rt_ / max(rc_, 1)
    rope_gbps = nr * (page + L * wl.n_kv_heads * d * 2) / (rope_ms * 1e-3) / 1e9
    # Delta re-RoPE leg: a second context in delta mode over the same pages; the
    # view alternates between the selection and the selection without its first
    # block, so every resident block is rotated in place by +-32 positions
    delta = None
    if args.delta_steps > 0:
        ws.ctx.kvm_ctx_evict(0, wl.final_blocks)
        dctx = k.KvmCtx(ws.dims, ws.dt, ws.k_view, ws.v_view, None, ws.k_view.shape[0],
                        wl.final_blocks, (wl.budget_blocks + wl.reserve_blocks) * wl.block_tokens,
                        wl.theta, wl.rope_layout, 64, 0, 1 << 20)
        for i, b in enumerate(ws.hits):
            dctx.kvm_ctx_set_source(int(b), 1, ws.hit_k[i], ws.hit_v[i], page, k.KVM_SRC_DEVICE)
        for i, b in enumerate(ws.misses):
            dctx.kvm_ctx_set_source(int(b), 1, ws.miss_k_d[i], ws.miss_v_d[i], page,
                                    k.KVM_SRC_DEVICE)
        sel_a = ws.sel[:n].clone()
        sel_b = ws.sel[1:n].clone()
        n_a = torch.tensor([n], dtype=torch.int32, device=dev)
        n_b = torch.tensor([n - 1], dtype=torch.int32, device=dev)
        dctx.kvm_rematerialize(sel_a, n_a, ws.page)
        torch.cuda.synchronize()
        k.kvm_profile_enable(True)
        dst = None
        for t in range(args.delta_steps):
            dst = dctx.kvm_rematerialize(sel_b if t % 2 == 0 else sel_a,
                                         n_b if t % 2 == 0 else n_a, ws.page)
        torch.cuda.synchronize()
        dc, dt_ = k.kvm_profile_read().get("remat", (0, float("nan")))
        k.kvm_profile_enable(False)
        dctx.close()
        d_ms = dt_ / max(dc, 1)
        d_bytes = dst["deltas"] * 2 * page
        delta = {"avg_ms": d_ms, "deltas_per_call": dst["deltas"], "bytes": d_bytes,
                 "GBps": d_bytes / (d_ms * 1e-3) / 1e9,
                 "hbm_frac": d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "traffic": traffic_for(traffic, *REMAT_DELTA_KERNEL)}
        log(f"delta leg: {d_ms:.2f} ms per remat, {dst['deltas']} blocks shifted in place")
        ws.reset_pool()
    fp8 = fp8_leg(k, ws, wl, dev, args.steps) if args.fp8 else None
    fp8s = fp8_scores_leg(k, ws, wl, dev, args.steps, args.warmup) if args.fp8 else None
    med = None
    if args.median_runs > 0:
        log(f"kernel medians over {args.median_runs} runs")
        med = kernel_medians(k, ws, args.median_runs, remat_bytes)
    cpu = None
    if args.cpu_baseline:
        log("timing the CPU oracle sample")
        cpu = cpu_baseline(wl, args.cpu_pairs)
    out = {
        "metric": METRIC if args.workload == "ws1m" else METRIC.replace("1M-tok", args.workload),
        "value": N / (ms * 1e-3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": workload_desc(wl),
                   "n_blocks": N, "n_q_tokens": T, "budget_blocks": wl.budget_blocks},
        "roofline": roof,
        "rooflines_other": others,
        "peaks_measured": peaks,
        "cpu_baseline": cpu,
        "kernel_medians": med,
        "remat": {"avg_ms": remat["per_step_ms"] if remat else None, "bytes": remat_bytes,
                  "GBps": remat_gbps,
                  "hbm_frac": remat_gbps / HBM_PEAK_GBPS if remat_gbps else None,
                  "hits": nh, "misses": nm},
        "score": {"ms": sum(v["avg_ms"] for kk, v in kern.items() if kk.startswith("score")),
                  "blocks_per_s": None, "tflops_per_pass": flops_pass / 1e12},
        "build": ({"blocks": med["build_blocks"], "avg_ms": med["build_ms"],
                   "GBps": med["build_GBps"], "hbm_frac": med["build_hbm_frac"],
                   "how": "one launch over raw K already in HBM, median of timed launches"}
                  if med else {}) | {
            "setup": {"blocks": bst["blocks"], "launches": bst["launches"], "GBps": build_gbps,
                      "hbm_frac": build_gbps / HBM_PEAK_GBPS,
                      "how": "the index build of the setup: 1024-block launches, each after "
                             "its chunk of raw K is drawn on the host and copied in"}},
        "build_rope": {"blocks": nr, "avg_ms": rope_ms, "GBps": rope_gbps,
                       "hbm_frac": rope_gbps / HBM_PEAK_GBPS},
        "delta_rerope": delta,
        "fp8_pages": fp8,
        "fp8_scores": fp8s,
        "pcie_leg": pcie,
        "whole_step_host_tier": None if pcie is None else {
            "workload": workload_desc(wl).split(":")[0] + ": the value step with the missing "
                        "half's raw K/V in pinned host memory (fetched H2D on side streams, "
                        "overlapped with the re-RoPE of the resident half)",
            "ms_per_step": pcie["ms_per_step"], "blocks_per_s": pcie["blocks_per_s"],
            "h2d_bytes": pcie["h2d_bytes"], "step_h2d_GBps": pcie["step_h2d_GBps"]},
        "kernels": kern,
    }
    if med:
        bgb = med["build_GBps"]
        others.append({"kernel": "build_index", "bound": "hbm", "achieved": bgb,
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": bgb / HBM_PEAK_GBPS,
                       "frac_of_measured": bgb / peaks["copy_kernel_GBps"],
                       # the counters were taken on the setup's 1024-block launches, not
                       # on this launch; their bytes per block are in the profile summary
                       "traffic": None})
    out["score"]["blocks_per_s"] = N / (out["score"]["ms"] * 1e-3)
    # (block, layer, KV head) index rows scored per second, and exps per second
    # over both passes (one per score and pass)
    out["score"]["rows_per_s"] = N * L * wl.n_kv_heads / (out["score"]["ms"] * 1e-3)
    out["score"]["exps_per_s"] = 2.0 * L * Hq * T * N / (out["score"]["ms"] * 1e-3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
