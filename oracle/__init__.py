"""fp64 CPU oracle of the Kara window-compression step (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's cpu_baseline
leg may import this package; the product path never does.
"""
from .kara_oracle import (  # noqa: F401
    Selection,
    batch_unit_scores,
    chunk_bound,
    compact_paged_sequence,
    compact_window_rows,
    compress_step,
    gather_window_rows,
    paged_decode_attention,
    rewrite_block_table,
    token2chunk_bridge_select,
    token2chunk_select,
    window_scores,
)
