"""Plain, slow, obviously correct CPU oracle of the KVMem working-set update.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The library under
``attention_space_block_amd`` never imports it and shares no code with it;
the two meet only in the seeded input generator ``synth``.

Every function computes in float64 (NumPy) and follows one passage of the
KVMem paper ("Virtualizing Million-Token Agent Workspaces on a Consumer
GPU"), cited in its docstring, or one RoPE identity of the InferScale paper
(Sec. 2.4 and Theorem 6). The paper's displayed equations were lost in the
extracted text; each function states the reading of the surrounding prose it
implements.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: closed forms, invariants, a textbook routine on a special case, brute
force on tiny inputs, or numbers printed on the pages (tests/golden/).
Parity unpinned: whether the scoring rule is *exactly* the paper's lost
Eq. (10) (only the prose survives), and whether the paper's engine used base
10000 and interleaved RoPE pairs; both readings are fixed here and stated.
"""
from .numerics import bf16_round, bf16_bits, round_to_dtype  # noqa: F401
from .meank import mean_k, mean_k_index, mean_k_from_rope  # noqa: F401
from .scores import block_scores, block_scores_streamed, lg_partial_scores  # noqa: F401
from .select import select_blocks, compact_positions, cutoff_margin  # noqa: F401
from .rope import rope_frequencies, rope_rotate, rope_matrix, bounded_delta_rope  # noqa: F401
from .plan import working_set_delta, PagePool, PoolFull  # noqa: F401
from .accounting import kv_bytes, index_bytes  # noqa: F401
from .tier import simulate_host_tier  # noqa: F401
