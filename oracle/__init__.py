"""CPU oracle for the N-gram embedding layer: test infrastructure, never the product path.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
"""
from .ngram_oracle import (  # noqa: F401
    PAD_ID, num_subtables, subtable_order, check_config, context, ngram_value, hash_indices,
    embed_from_indices, table_fetch, prefill, DecodeOracle, param_count, AMP_MODES, amplify,
    backward, embed_basic, backward_basic, hash_slot_stats,
)
