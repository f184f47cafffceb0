"""Byte accounting of raw KV and of the Mean-K index.

InferScale paper, Sec. 3.5 (storage cost): a span of c tokens stores
2 * L * c * h * d * b bytes of KV (layers L, KV heads h, head dim d, b bytes
per element). KVMem paper, Sec. 4.3 and Table 4: the Mean-K index keeps one
vector per (block, indexed layer, KV head), so it grows linearly in blocks.
"""


def kv_bytes(n_layers: int, n_tokens: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * n_layers * n_tokens * n_kv_heads * head_dim * elem_bytes


def index_bytes(n_blocks: int, n_layers: int, n_kv_heads: int, head_dim: int,
                elem_bytes: int) -> int:
    return n_blocks * n_layers * n_kv_heads * head_dim * elem_bytes
