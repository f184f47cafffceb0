"""The five seeded synthetic workspaces and the knobs that shape them.

Shapes follow the KVMem paper ("Virtualizing Million-Token Agent Workspaces on
a Consumer GPU"): 32-token logical blocks (Sec. 4.3), always-kept sink and
recent blocks plus a top-k remainder within a token budget (Sec. 4.3), a 1M
workspace with a 128K selection budget and a 64K generation reserve (the
DeepSWE setting, Sec. 6.6), and a 10M workspace with a 64K view (Table 4).
The value laws (unit-variance noise plus per-block offsets) are stand-ins:
the pages give no distribution for real K.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# Generator stream ids (the "tensor" field of the counter key).
TENSOR = {
    "K": 1,        # raw pre-RoPE K noise
    "V": 2,        # raw V noise
    "KOFF": 3,     # per-(block, layer, KV head) K offset vectors
    "VOFF": 4,     # per-(block, layer, KV head) V offset vectors
    "Q": 5,        # query noise (single-step workloads)
    "IDX": 6,      # noise of a directly drawn index
    "SCORE": 9,    # synthetic score vectors for selection tests
    "UINIT": 10,   # churn: initial topic vector
    "QSTEP": 1000,  # churn: query noise of step t uses QSTEP + t
    "WSTEP": 2000,  # churn: topic innovation of step t uses WSTEP + t
}


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    dtype: str            # "f32", "bf16" or "fp8" (E4M3): the dtype of raw K/V (and of the
                          # index and q, which are bf16 for fp8 K/V)
    n_blocks: int         # history blocks at the (first) scoring step
    n_q_tokens: int
    n_sink: int
    n_recent: int
    budget_blocks: int
    block_tokens: int = 32
    seed: int = 0
    off_sigma: float = 0.0      # std of the per-block offset vectors
    theta: float = 10000.0
    rope_layout: int = 0        # 0 interleaved pairs (2t, 2t+1); 1 half-split (t, t+d/2)
    index_direct: bool = False  # index drawn directly (raw K never materialised)
    planted_block: int = -1     # tiny case: block whose Mean-K is planted in q
    planted_gain: float = 3.0
    steps: int = 1              # churn: number of agent steps
    append_blocks: int = 0      # churn: blocks appended per step
    topic_rho: float = 0.0      # churn: AR(1) correlation of the query topic
    topic_scale: float = 0.0    # churn: per-element std of the query topic
    reserve_blocks: int = 0     # generation reserve (sizes the pool only)
    tile_blocks: int = 512      # host-tiled scoring: blocks per tile

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def index_dtype(self) -> str:
        """dtype of the Mean-K index and the queries: bf16 when K/V are fp8."""
        return "bf16" if self.dtype == "fp8" else self.dtype

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def block_elems(self) -> int:
        """Elements of one raw K (or V) block, all layers and KV heads."""
        return self.n_layers * self.n_kv_heads * self.block_tokens * self.head_dim

    @property
    def block_bytes(self) -> int:
        return self.block_elems * self.elem_bytes

    @property
    def index_row_bytes(self) -> int:
        return self.head_dim * (4 if self.index_dtype == "f32" else 2)

    @property
    def final_blocks(self) -> int:
        return self.n_blocks + max(0, self.steps - 1) * self.append_blocks

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 4096-token history, one query token planted on block 64's Mean-K.
    "tiny": Workload("tiny", 1, 2, 4, 64, "f32", 128, 1, 1, 2, 11,
                     planted_block=64, planted_gain=3.0),
    # 64K-token history, offsets with std 0.5, 256 query tokens, 16K budget.
    "ctx64k": Workload("ctx64k", 8, 8, 48, 128, "bf16", 2048, 256, 1, 64, 512,
                       off_sigma=0.5),
    # 1M-token workspace, 512 query tokens, 128K budget, 64K reserve.
    "ws1m": Workload("ws1m", 64, 8, 48, 128, "bf16", 32768, 512, 1, 64, 4096,
                     off_sigma=0.5, reserve_blocks=2048),
    # 10M-token workspace, directly drawn index, decode-style single query.
    "ws10m": Workload("ws10m", 64, 8, 48, 128, "bf16", 312500, 1, 1, 256, 2048,
                      off_sigma=0.5, index_direct=True, tile_blocks=512),
    # 1M-token workspace run for 32 agent steps, +64 blocks per step.
    "churn": Workload("churn", 64, 8, 48, 128, "bf16", 32768, 512, 1, 64, 4096,
                      off_sigma=0.5, steps=32, append_blocks=64,
                      topic_rho=0.9, topic_scale=0.35, reserve_blocks=2048),
}
# The churn workspace with 4 layers and 8 steps: the same history, queries,
# budget and step structure at 1/16 of the scoring work, so the CPU oracle can
# produce every step's expected selection.
WORKLOADS["churn_l4"] = WORKLOADS["churn"].scaled(name="churn_l4", n_layers=4, steps=8)
# FP8 (E4M3) K/V pages, as the pages' engine runs its KV cache: the same values
# as the bf16 workspaces, rounded to FP8 instead of bf16; index and q stay bf16.
WORKLOADS["ctx64k_fp8"] = WORKLOADS["ctx64k"].scaled(name="ctx64k_fp8", dtype="fp8")
WORKLOADS["ws1m_fp8"] = WORKLOADS["ws1m"].scaled(name="ws1m_fp8", dtype="fp8")


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
