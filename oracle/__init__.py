"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .bi_oracle import (  # noqa: F401
    IGNORE_INDEX, STAT_FIELDS, backward, backward_rows, brute_force, chunk_stats,
    combine, decode, forward, forward_batch, label_kind, policy_terms, row_statistics,
)
