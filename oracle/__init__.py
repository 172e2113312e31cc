"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .bi_oracle import (  # noqa: F401
    IGNORE_INDEX, STAT_FIELDS, backward, backward_rows, brute_force, chunk_stats,
    combine, decode, diff_stats, forward, forward_batch, forward_multi, label_kind, lmhead_backward,
    lmhead_logits, lmhead_tile_stats, policy_terms,
    row_statistics,
)
