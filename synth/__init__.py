"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks."""

from .gen import (  # noqa: F401
    BLOCK_ROWS,
    CONFIGS,
    InputSpec,
    duplicate_pairs,
    gen_attention_inputs,
    gen_keys,
    gen_q_rows,
    gen_w_rows,
    make_inputs,
    mxfp4_quantize,
    sample_rows,
)
