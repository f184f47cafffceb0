"""Step-level working-set update over the C ABI.

KVMem (Sec. 4.2) updates the historical working set once per agent step,
after the step's prefill and before decoding: the step's freshly completed
blocks are indexed (Sec. 5, incremental indexing) and registered as resident,
every indexed block is scored against the step's queries, the selection is
made and the execution view is rematerialized (Sec. 4.3, 4.4). This class
owns the device buffers of that loop (index, score workspace, selection, page
pool) and calls the four library entry points in order; it performs no
arithmetic of its own.
"""
from __future__ import annotations

from . import api
from .api import KVM_INDEX_DEVICE


class WorkingSetUpdater:
    def __init__(self, dims: api.Dims, dtype: int, index_cap: int, budget_blocks: int,
                 n_sink: int, n_recent: int, n_slots: int, max_pos: int, device,
                 rope_theta: float = 10000.0, rope_layout: int = 0, batch_blocks: int = 64,
                 staging_blocks: int = 0, delta_limit: int = 0):
        import torch
        self.dims, self.dtype = dims, dtype
        self.cap, self.budget = index_cap, budget_blocks
        self.n_sink, self.n_recent = n_sink, n_recent
        self.dev = device
        # page elements in the K/V dtype; the index and queries are bf16 for FP8 K/V
        tdt = {api.KVM_F32: torch.float32, api.KVM_BF16: torch.int16,
               api.KVM_FP8_E4M3: torch.uint8}[dtype]
        self.index_dtype = api.KVM_BF16 if dtype == api.KVM_FP8_E4M3 else dtype
        self.elem_dtype = tdt
        self.block_elems = dims.n_layers * dims.n_kv_heads * dims.block_tokens * dims.head_dim
        self.block_bytes = self.block_elems * tdt.itemsize
        self.index = torch.zeros((dims.n_layers, dims.n_kv_heads, index_cap, dims.head_dim),
                                 dtype=torch.float32 if dtype == api.KVM_F32 else torch.int16,
                                 device=device)
        self.k_view = torch.zeros((n_slots, self.block_elems), dtype=tdt, device=device)
        self.v_view = torch.zeros((n_slots, self.block_elems), dtype=tdt, device=device)
        # bounded delta re-RoPE (delta_limit > 0) keeps no raw-K shadow pages
        self.k_shadow = (None if delta_limit > 0 else
                         torch.zeros((n_slots, self.block_elems), dtype=tdt, device=device))
        self.ctx = api.KvmCtx(dims, dtype, self.k_view, self.v_view, self.k_shadow, n_slots,
                              index_cap, max_pos, rope_theta, rope_layout, batch_blocks,
                              staging_blocks, delta_limit)
        self.sel = torch.empty(budget_blocks, dtype=torch.int32, device=device)
        self.n_sel = torch.empty(1, dtype=torch.int32, device=device)
        self.base_pos = torch.empty(budget_blocks, dtype=torch.int32, device=device)
        self.page_table = torch.empty(budget_blocks, dtype=torch.int32, device=device)
        self.scores = torch.empty(index_cap, dtype=torch.float32, device=device)
        self.sel_ws = torch.empty(api.kvm_select_ws_bytes(index_cap), dtype=torch.uint8,
                                  device=device)
        self.ws = None
        self.ws_key = None
        self.n_blocks = 0

    def build(self, k_raw, first_block: int, n_blocks: int, block_stride: int | None = None):
        """Index rows [first_block, first_block + n_blocks) from device raw K."""
        api.kvm_build_index(self.dims, self.dtype, k_raw, block_stride or self.block_bytes,
                            first_block, n_blocks, self.index, self.cap)
        self.n_blocks = max(self.n_blocks, first_block + n_blocks)

    def append(self, k_raw, v_raw, n_blocks: int, block_stride: int | None = None):
        """The step's freshly prefilled blocks: index them and register them as
        GPU-resident pages."""
        first = self.n_blocks
        self.build(k_raw, first, n_blocks, block_stride)
        self.ctx.kvm_ctx_register_resident(first, n_blocks, k_raw, v_raw,
                                           block_stride or self.block_bytes)
        return first

    def _workspace(self, n_q_tokens: int):
        import torch
        key = (n_q_tokens, self.n_blocks)
        if self.ws_key != key:
            nbytes = api.kvm_score_ws_bytes(self.dims, self.index_dtype, n_q_tokens, self.n_blocks)
            if self.ws is None or self.ws.numel() < nbytes:
                self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
            self.ws_key = key
        return self.ws

    def score(self, q, n_q_tokens: int):
        ws = self._workspace(n_q_tokens)
        api.kvm_score_blocks(self.dims, self.index_dtype, q, n_q_tokens, self.index, self.cap,
                             self.n_blocks, KVM_INDEX_DEVICE, 0, self.scores, ws, ws.numel())

    def select(self):
        api.kvm_select(self.scores, self.n_blocks, self.n_sink, self.n_recent, self.budget,
                       self.dims.block_tokens, self.sel, self.n_sel, self.base_pos,
                       self.sel_ws, self.sel_ws.numel())

    def rematerialize(self) -> dict:
        return self.ctx.kvm_rematerialize(self.sel, self.n_sel, self.page_table)

    def update(self, q, n_q_tokens: int) -> dict:
        """Score, select and rematerialize: the working-set update of one step."""
        self.score(q, n_q_tokens)
        self.select()
        return self.rematerialize()

    def close(self):
        self.ctx.close()
