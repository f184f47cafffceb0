"""Python names for the C entry points of include/kvm.h (marshalling only)."""
from __future__ import annotations

import ctypes

import numpy as np

from . import _abi
from ._abi import (  # noqa: F401
    Dims, KvmError, RematStats, KVM_F32, KVM_BF16, KVM_FP8_E4M3, KVM_INDEX_DEVICE,
    KVM_INDEX_HOST_TILED,
    KVM_SRC_NONE, KVM_SRC_HOST_PINNED, KVM_SRC_DEVICE,
    KVM_TIER_LRU, KVM_TIER_LRFU,
    KVM_RATE_COPY, KVM_RATE_MFMA_BF16, KVM_RATE_EXP, KVM_RATE_SCORE_MIX,
)


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def dims_for(wl) -> Dims:
    """kvm_dims of a workload description (anything with the five fields)."""
    return Dims(wl.n_layers, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.block_tokens)


def dtype_code(dtype: str) -> int:
    return {"f32": KVM_F32, "bf16": KVM_BF16, "fp8": KVM_FP8_E4M3}[dtype]


def kvm_version() -> int:
    return _abi.lib().kvm_version()


def kvm_build_index(dims: Dims, dtype: int, k_raw, k_block_stride: int, first_block: int,
                    n_blocks: int, index, index_cap_blocks: int, stream=None) -> None:
    rc = _abi.lib().kvm_build_index(ctypes.byref(dims), dtype, _ptr(k_raw), k_block_stride,
                                    first_block, n_blocks, _ptr(index), index_cap_blocks,
                                    _stream(stream))
    _abi.check(rc, "kvm_build_index")


def kvm_score_ws_bytes(dims: Dims, dtype: int, n_q_tokens: int, n_blocks: int,
                       index_loc: int = KVM_INDEX_DEVICE, tile_blocks: int = 0) -> int:
    return int(_abi.lib().kvm_score_ws_bytes(ctypes.byref(dims), dtype, n_q_tokens, n_blocks,
                                             index_loc, tile_blocks))


def kvm_score_blocks(dims: Dims, dtype: int, q, n_q_tokens: int, index, index_cap_blocks: int,
                     n_blocks: int, index_loc: int, tile_blocks: int, scores, ws, ws_bytes: int,
                     stream=None) -> None:
    rc = _abi.lib().kvm_score_blocks(ctypes.byref(dims), dtype, _ptr(q), n_q_tokens, _ptr(index),
                                     index_cap_blocks, n_blocks, index_loc, tile_blocks,
                                     _ptr(scores), _ptr(ws), ws_bytes, _stream(stream))
    _abi.check(rc, "kvm_score_blocks")


def kvm_quantize_e4m3(src, src_dtype: int, n: int, dst, stream=None) -> None:
    rc = _abi.lib().kvm_quantize_e4m3(_ptr(src), src_dtype, n, _ptr(dst), _stream(stream))
    _abi.check(rc, "kvm_quantize_e4m3")


def kvm_select_ws_bytes(n_blocks: int) -> int:
    return int(_abi.lib().kvm_select_ws_bytes(n_blocks))


def kvm_select(scores, n_blocks: int, n_sink: int, n_recent: int, budget_blocks: int,
               block_tokens: int, sel, n_sel, base_pos, ws=None, ws_bytes: int = 0,
               stream=None) -> None:
    rc = _abi.lib().kvm_select(_ptr(scores), n_blocks, n_sink, n_recent, budget_blocks,
                               block_tokens, _ptr(sel), _ptr(n_sel), _ptr(base_pos), _ptr(ws),
                               ws_bytes, _stream(stream))
    _abi.check(rc, "kvm_select")


def kvm_select_noalloc(scores, n_blocks: int, n_sink: int, n_recent: int, budget_blocks: int,
                       block_tokens: int, sel, n_sel, base_pos, stream=None) -> None:
    rc = _abi.lib().kvm_select_noalloc(_ptr(scores), n_blocks, n_sink, n_recent, budget_blocks,
                                       block_tokens, _ptr(sel), _ptr(n_sel), _ptr(base_pos),
                                       _stream(stream))
    _abi.check(rc, "kvm_select_noalloc")


def kvm_tier_simulate(policy: int, host_blocks: int, lam: float, steps) -> list:
    """Host-tier admission over a trace; steps = [(new, sel, miss), ...], each an
    ascending list of block ids. Returns [(host_hits, nvme_reads, demotions)]."""

    def csr(lists):
        off = np.zeros(len(lists) + 1, dtype=np.int64)
        off[1:] = np.cumsum([len(x) for x in lists])
        blk = np.ascontiguousarray(np.concatenate([np.asarray(x, dtype=np.int32).reshape(-1)
                                                   for x in lists] + [np.zeros(0, np.int32)]))
        return off, blk
    n = len(steps)
    arrs = [csr([st[i] for st in steps]) for i in range(3)]
    out = np.zeros((max(n, 1), 3), dtype=np.int32)
    pol = _abi.TierPolicy(policy, host_blocks, lam)
    ptr = lambda a: a.ctypes.data if a.size else None
    rc = _abi.lib().kvm_tier_simulate(ctypes.byref(pol), n, ptr(arrs[0][0]), ptr(arrs[0][1]),
                                      ptr(arrs[1][0]), ptr(arrs[1][1]), ptr(arrs[2][0]),
                                      ptr(arrs[2][1]), out.ctypes.data)
    _abi.check(rc, "kvm_tier_simulate")
    return [tuple(int(v) for v in row) for row in out[:n]]


def kvm_profile_enable(on: bool) -> None:
    _abi.check(_abi.lib().kvm_profile_enable(1 if on else 0), "kvm_profile_enable")


def kvm_profile_read() -> dict:
    """{kernel name: (launches, total_ms)} since profiling was enabled."""
    n = ctypes.c_int32()
    buf = (_abi.KernelStat * 64)()
    _abi.check(_abi.lib().kvm_profile_read(buf, 64, ctypes.byref(n)), "kvm_profile_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n.value, 64))}


def kvm_measure_rate(kind: int, n: int, scratch, stream=None) -> float:
    """Measured rate of one unit (see KVM_RATE_*); scratch: a device tensor."""
    out = ctypes.c_double()
    nbytes = scratch.numel() * scratch.element_size()
    rc = _abi.lib().kvm_measure_rate(kind, n, _ptr(scratch), nbytes, ctypes.byref(out),
                                     _stream(stream))
    _abi.check(rc, "kvm_measure_rate")
    return float(out.value)


class KvmCtx:
    """Owner of one kvm_ctx (block records, side stream, staging, RoPE table)."""

    def __init__(self, dims: Dims, dtype: int, k_view, v_view, k_shadow, n_slots: int,
                 max_blocks: int, max_pos: int, rope_theta: float = 10000.0,
                 rope_layout: int = 0, batch_blocks: int = 64, staging_blocks: int = 0,
                 delta_limit: int = 0):
        d = _abi.CtxDesc()
        d.dims = dims
        d.dtype = dtype
        d.rope_layout = rope_layout
        d.rope_theta = rope_theta
        d.max_pos = max_pos
        d.n_slots = n_slots
        d.k_view = _ptr(k_view)
        d.v_view = _ptr(v_view)
        d.k_shadow = _ptr(k_shadow)
        d.max_blocks = max_blocks
        d.batch_blocks = batch_blocks
        d.staging_blocks = staging_blocks
        d.delta_limit = delta_limit
        h = ctypes.c_void_p()
        _abi.check(_abi.lib().kvm_ctx_create(ctypes.byref(d), ctypes.byref(h)), "kvm_ctx_create")
        self._h = h
        # objects the library keeps pointers to: the pool pages for the ctx's
        # life, gather callbacks, and the lower-tier buffers of each recorded
        # block range (replaced when the same range is recorded again)
        self._keep = [k_view, v_view, k_shadow]
        self._sources = {}

    def close(self):
        if self._h:
            _abi.lib().kvm_ctx_destroy(self._h)
            self._h = None
        self._keep = []
        self._sources = {}

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def kvm_ctx_set_source(self, first_block: int, n_blocks: int, k_base, v_base,
                           block_stride: int, loc: int) -> None:
        rc = _abi.lib().kvm_ctx_set_source(self._h, first_block, n_blocks, _ptr(k_base),
                                           _ptr(v_base), block_stride, loc)
        _abi.check(rc, "kvm_ctx_set_source")
        self._sources[(first_block, n_blocks)] = (k_base, v_base)

    def kvm_ctx_set_gather(self, first_block: int, n_blocks: int, fn) -> None:
        """fn(block, which, dst_ptr) -> int, called from library worker threads."""
        cb = _abi.GATHER_FN(lambda user, b, which, dst: int(fn(int(b), int(which), int(dst))))
        self._keep.append(cb)
        rc = _abi.lib().kvm_ctx_set_gather(self._h, first_block, n_blocks, cb, None)
        _abi.check(rc, "kvm_ctx_set_gather")

    def kvm_ctx_set_gather_raw(self, first_block: int, n_blocks: int, fn_ptr: int,
                               user_ptr: int) -> None:
        """Same as kvm_ctx_set_gather with a C function pointer (no Python in
        the gather path); the caller keeps `user_ptr` alive."""
        cb = ctypes.cast(ctypes.c_void_p(fn_ptr), _abi.GATHER_FN)
        self._keep.append(cb)
        rc = _abi.lib().kvm_ctx_set_gather(self._h, first_block, n_blocks, cb,
                                           ctypes.c_void_p(user_ptr))
        _abi.check(rc, "kvm_ctx_set_gather")

    def kvm_ctx_register_resident(self, first_block: int, n_blocks: int, k_raw, v_raw,
                                  block_stride: int, stream=None) -> None:
        rc = _abi.lib().kvm_ctx_register_resident(self._h, first_block, n_blocks, _ptr(k_raw),
                                                  _ptr(v_raw), block_stride, _stream(stream))
        _abi.check(rc, "kvm_ctx_register_resident")

    def kvm_ctx_register_resident_list(self, blocks, k_raw, v_raw, block_stride: int,
                                       stream=None) -> None:
        """blocks: strictly ascending block ids (any int sequence); the raw K/V
        of blocks[i] at k_raw / v_raw + i * block_stride."""
        ids = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
        rc = _abi.lib().kvm_ctx_register_resident_list(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), ids.size, _ptr(k_raw), _ptr(v_raw),
            block_stride, _stream(stream))
        _abi.check(rc, "kvm_ctx_register_resident_list")

    def kvm_ctx_build_index_rope(self, k_rope, block_stride: int, first_block: int,
                                 n_blocks: int, pos0: int, index, index_cap_blocks: int,
                                 stream=None) -> None:
        rc = _abi.lib().kvm_ctx_build_index_rope(self._h, _ptr(k_rope), block_stride,
                                                 first_block, n_blocks, pos0, _ptr(index),
                                                 index_cap_blocks, _stream(stream))
        _abi.check(rc, "kvm_ctx_build_index_rope")

    def kvm_rematerialize(self, sel, n_sel, page_table, stream=None) -> dict:
        st = RematStats()
        rc = _abi.lib().kvm_rematerialize(self._h, _ptr(sel), _ptr(n_sel), _ptr(page_table),
                                          ctypes.byref(st), _stream(stream))
        _abi.check(rc, "kvm_rematerialize")
        return st.as_dict()

    def kvm_ctx_block_deltas(self, block: int) -> int:
        n = ctypes.c_int32()
        _abi.check(_abi.lib().kvm_ctx_block_deltas(self._h, block, ctypes.byref(n)),
                   "kvm_ctx_block_deltas")
        return int(n.value)

    def kvm_ctx_evict(self, first_block: int, n_blocks: int) -> None:
        _abi.check(_abi.lib().kvm_ctx_evict(self._h, first_block, n_blocks), "kvm_ctx_evict")

    def kvm_ctx_sync(self) -> None:
        _abi.check(_abi.lib().kvm_ctx_sync(self._h), "kvm_ctx_sync")

    def kvm_ctx_set_serialized(self, on: bool) -> None:
        _abi.check(_abi.lib().kvm_ctx_set_serialized(self._h, 1 if on else 0),
                   "kvm_ctx_set_serialized")

    def kvm_ctx_block_state(self, block: int):
        s, p = ctypes.c_int32(), ctypes.c_int32()
        _abi.check(_abi.lib().kvm_ctx_block_state(self._h, block, ctypes.byref(s), ctypes.byref(p)),
                   "kvm_ctx_block_state")
        return s.value, p.value
