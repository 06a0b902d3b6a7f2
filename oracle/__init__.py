"""CPU oracle for the approximate-attention prefill path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the product library.
"""
from .spava_oracle import (  # noqa: F401
    split_sequence, block_scores, context_block_scores, kv_overlap, select_passing, gather_passing, attend,
    anchor_rows, context_rows, query_partials, lse_merge, approx_prefill,
    sampled_rows, dense_causal,
)
