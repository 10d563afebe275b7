"""CPU oracle of the MSA hot path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never uses it.
"""
from .msa_oracle import (  # noqa: F401
    SelectResult,
    attention_backward,
    attention_forward,
    block_max_scores,
    gemma_rmsnorm,
    index_select,
    indexer_features,
    key_set,
    qk_norm_rope_backward,
    qk_norm_rope_forward,
    rope_cos_sin,
    rope_rotate_half,
    round_to_bf16,
    select_row,
    selection_valid_within_ties,
    selectors_of_block,
    sequence_layout,
)
