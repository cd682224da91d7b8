"""Float64 CPU oracle for attention over a context-parallel striped paged KV pool.

TEST INFRASTRUCTURE. Nothing on the product path may import, call or execute anything in this package: only the test
suite, the smoke check of the build entry point and the CPU-baseline leg of the benchmark use it. It shares no code
with the HIP library (no kernels, headers, helpers, tables or constants); both sides take their inputs from the seeded
generators in ``workloads``.

What it states, and where the pages state it:

* ``slots``: the placement rule for a context-parallel pool and the per-rank write view with the sink page
  (mstar PR #1124, "Context / Sequence Parallel 1/5: split the KV cache by position across GPUs (DCP)",
  PR description and commit message).
* ``attn``: softmax attention with its natural-log log-sum-exp; the per-stripe partial (each rank attends its own
  slots and returns the partial with its LSE); the exact LSE merge of partials; own-token causal attention over the
  in-step K/V; the whole row as plain attention over the unstriped logical KV (same PR; and the vLLM compare view
  "[Core] Add explicit layer parallel plans", ``FlashAttentionImpl._forward_with_dcp``).
* ``quant``: what an fp8 pool's codes stand for (per-tensor k_descale / v_descale passed to the attention calls in
  the same vLLM compare view; the code format is a reading, stated there).

Every function is pinned by CPU tests (``tests/test_oracle_*.py``) against brute force, closed forms, invariants
and library routines; none is "parity unpinned".
"""
from .slots import slot_map, slot_map_rank, stripe_positions, stripe_len, place_logical_rows, gather_stripe
from .attn import (attention, gqa_attention, stripe_partial, merge, own_token_partial, row_attention,
                        row_partials, NEG_INF)
from .quant import e4m3_value, dequantize_e4m3

__all__ = [
    "slot_map", "slot_map_rank", "stripe_positions", "stripe_len", "place_logical_rows", "gather_stripe",
    "attention", "gqa_attention", "stripe_partial", "merge", "own_token_partial", "row_attention", "row_partials",
    "NEG_INF", "e4m3_value", "dequantize_e4m3",
]
