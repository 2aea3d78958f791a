"""CPU oracle for prompt-deduplicated split attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``shared_prompt_dedup_amd``) never does, and this package imports nothing
from it.  The two share no code: only the seeded input generators in
``workloads.py`` serve both.

Everything is numpy, integer work exact and floating point in fp64.  Each
function names the passage of the pages it follows:

* "How Prompt Deduplication Works" -- Phase 1 (Prompt Detection &
  Deduplication), Phase 2 (Split Attention Optimization), Phase 3
  (Transparent Reconstruction), Core Algorithm: ZoRRoTrain Class (Finding
  Prompt Groups, Creating Deduplicated Batch, Reconstructing Original Batch),
  Working with Packed/Unpacked Sequences, Correctness & Gradients;
* "Performance Benchmarks" -- Redundancy Analysis, Testing Correctness and
  Performance (outputs and gradients are validated against a
  non-deduplicated reference).

The attention oracle is deliberately the NON-deduplicated computation: plain
causal attention run separately on every ``[prompt][response]`` sample, then
mapped onto the packed rows.  Pins (tests/test_oracle_*.py) tie each function
to something other than itself: the pages' worked examples, brute force,
closed forms, a library attention routine, autograd and finite differences.
"""
from .dedup import (find_prompt_groups, find_shared_prefix, create_deduplicated_batch, reconstruct_sequences,
                    pack_rows, reconstruct_backward, pack_rows_backward, sample_rows, redundancy_counts,
                    attention_mask_to_flash_attn_params, varlen_params)
from .attention import (split_attention_forward, split_attention_backward,
                        forward_rows, dq_rows, dkdv_rows, attended_pairs)

__all__ = [
    "find_prompt_groups", "find_shared_prefix", "create_deduplicated_batch", "reconstruct_sequences", "pack_rows",
    "reconstruct_backward", "pack_rows_backward", "sample_rows", "redundancy_counts",
    "attention_mask_to_flash_attn_params", "varlen_params",
    "split_attention_forward", "split_attention_backward", "forward_rows", "dq_rows",
    "dkdv_rows", "attended_pairs",
]
