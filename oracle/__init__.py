"""fp64 CPU oracle for the FlashBlock attention step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (the ``cached_attention_amd`` package and its HIP library) never
imports, links or runs this package, and this package never imports the product
path: the two share no code.  Inputs come from ``cached_attention_amd.workloads``
(seeded draws only, no attention arithmetic) or from the tests themselves.

Source of what is computed: the FlashBlock pages -- the explainer page
"FlashBlock: Attention Caching for Efficient Long-Context Block Diffusion"
(Technical Summary section 2, "Core Mechanism", its merge equation, and
"Adaptive Reuse Strategies") and the FlashBlock abstract.  Where the pages
leave a step open, the reading taken is stated at the function that takes it.

Pins (tests/test_oracle_pins.py): brute force on tiny inputs, the CPU fp64
``scaled_dot_product_attention`` and ``logsumexp`` library routines (with their
own GQA convention), hand-derived worked examples under ``tests/golden/``,
closed forms (zero keys, constant values, a single key, score shifts, key
permutations), the partition invariant of the merge, cached mode at r = 1
against full recompute, and the refresh schedule.  The adaptive reuse policies
(``policies.py``) are pinned by constructed update counts and similarities,
their extreme thresholds against full recompute and against never refreshing,
and a per-head partition of given masks.  Sparse attention without the
residual (``sparse_only_step``) is pinned by its two extremes, every chunk
selected (the library routine over the whole prefix) and none (over the block
alone), and by brute force over the selected tokens.  The block append is pinned against
direct concatenation, and chunk selection by constructed pooled means, the
max over a KV group's queries, ties to the lower index and a brute-force
check of the kept set.  Cached mode at r > 1, the sparse residual and the policies'
per-head reuse are pinned by their closed form: one softmax over all keys in
which each prefix key is scored against the query of the step that last
refreshed it and each block (or selected-chunk) key against the current query,
written out by brute force.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    partial_attention,
    merge,
    kv_group,
    prefix_token_sets,
    prefix_partial,
    block_partial,
    merge_outputs,
    full_step,
    run_block,
    refresh_due,
    to_output_layout,
    sparse_only_step,
    grow_prefix,
    append_block_rows,
    BlockResult,
)
from .policies import (  # noqa: F401
    updated_tokens,
    tau_mask,
    head_similarity,
    gamma_mask,
    run_block_policy,
    pooled_chunk_keys,
    chunk_scores,
    select_chunks,
)
