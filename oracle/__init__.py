"""CPU oracle of the lightning-indexer top-k step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library.
"""

from .indexer import (  # noqa: F401
    E2M1_TABLE,
    E4M3FN_TABLE,
    bf16_bits_to_f64,
    e4m3fn_bits_to_f64,
    e8m0_bits_to_f64,
    mxfp4_bits_to_f64,
    indexer_topk,
    materialized_score_bytes,
    score_error_bound,
    score_row,
    score_rows,
    select_topk,
    total_visible_pairs,
    visible_count,
)
from .quant import E4M3_MAX, e4m3fn_encode_rne, quantize_q_e4m3  # noqa: F401,E402
from .two_stage import block_keys_mean, f32_to_bf16_bits_rne, two_stage_topk  # noqa: F401,E402
from .attention import attention_error_bound, default_scale, sparse_attention  # noqa: F401,E402
