"""Seeded synthetic inputs for tree-verify attention and greedy acceptance.

This package only draws random numbers, tree shapes and raw storage bytes.
It holds none of the arithmetic of the method (no dequantisation, no
attention, no argmax), so both the CPU oracle and the GPU path can consume
what it returns without sharing any of the computation under test.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Q4_0_BLOCK,
    Q4_0_BLOCK_BYTES,
    q4_0_row_bytes,
    streams,
    q4_0_cache,
    f16_cache,
    f16_normal,
    draft_tree,
    chain_tree,
    sibling_distinct_tokens,
    planted_logits,
    attn_inputs,
    full_step_tree,
    full_step_cache,
    full_step_qkv,
    full_step_layer,
)
