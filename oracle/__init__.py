"""CPU oracle for the DSA lightning-indexer selection path (test infrastructure).

This package is a plain, slow, fp64 NumPy statement of what the selection
path computes.  It exists to check the HIP library and is used only by
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``; the product path never imports or calls it.  It shares no code
with the HIP library (only the seeded input generators in ``synthetic``).

Pins: every function here is checked against something other than itself in
``tests/test_oracle_pins.py`` (exact-rational brute force on tiny inputs,
hand-computed fixtures under ``tests/golden/``, closed forms, special cases
and invariants).  No function is parity-unpinned.
"""
from .indexer import (  # noqa: F401
    visible_keys,
    head_scores,
    rank_desc,
    select_topk,
    score_topk,
    score_topk_packed,
    scores_at_indices,
    indexer_backward,
    indexer_backward_packed,
    round_to_bf16,
    k_norm,
    pool_count,
    kpool_compress,
    pooled_index_scores,
    visible_pools,
    topk_pools,
    expand_selection,
)
