"""CPU oracle of the lightning-indexer top-k step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library.
"""

from .indexer import (  # noqa: F401
    E4M3FN_TABLE,
    bf16_bits_to_f64,
    e4m3fn_bits_to_f64,
    indexer_topk,
    materialized_score_bytes,
    score_error_bound,
    score_row,
    score_rows,
    select_topk,
    total_visible_pairs,
    visible_count,
)
