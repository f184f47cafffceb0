"""Seeded synthetic workspaces: the inputs shared by the oracle and the HIP path.

Nothing in this package computes a step of the retrieval method (no block
mean, score, selection or rotation). It only draws raw pre-RoPE K/V blocks,
query vectors, directly drawn indexes and score vectors from a counter-based
generator, so that any block can be regenerated from (seed, tensor, block)
alone. The generator is defined in ``gen.c``; ``reference.py`` restates it in
NumPy and the CPU tests pin the two against each other.
"""
from .workloads import Workload, WORKLOADS, get_workload, TENSOR  # noqa: F401
from .generate import (  # noqa: F401
    kv_blocks,
    query,
    index_direct,
    churn_shift,
    unit_stream,
    scores_f32,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    stream_key,
    gather_store,
)
