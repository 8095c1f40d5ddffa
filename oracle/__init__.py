"""fp64 CPU oracle for the latent-attention (LAGA-style MLA) block.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain definition that
the GPU library is checked against. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library itself never
does, and this package imports nothing from the library.

What it follows: the LAGA paper's abstract ("A Training-Memory Regression in
MLA Sequence Parallelism: Why Megatron-Core Forbids Absorption, and LAGA -- a
Communication-Efficient Fix", weekinpapers.com and OpenAlex pages, Abstract)
says that LAGA keeps the latent-only gather, rebuilds each head's K and V
locally from the gathered latent, and is then exactly the explicit MLA form
(bit-identical at one sequence-parallel rank). So the oracle is explicit MLA
written out: up-project the latent per head, then masked softmax attention.

Parity status: every function here is pinned by tests that do not re-type
its formulas (brute-force loops, the absorbed reformulation, textbook causal
attention through a library routine, closed-form special cases, finite
differences, shard and segment identities). None is "parity unpinned".
"""

from .mla_oracle import (  # noqa: F401
    default_scale,
    segment_start,
    row_positions,
    visible_range,
    visible_pairs,
    key_range,
    keys_needed,
    mla_forward,
    mla_backward,
    mla_forward_absorbed,
    attention_flops,
)
