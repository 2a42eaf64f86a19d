"""MI355X (gfx950) lightning-indexer top-k: streaming scoring + partition-merge top-k.

The compute path is ``libsi_indexer.so`` (hand-written HIP kernels behind a C ABI,
``include/si_indexer.h``); this package only marshals torch tensors into it.  Importing
it loads the library and fails if it has not been built.
"""

from . import _lib
from .api import (  # noqa: F401
    Plan,
    TwoStagePlan,
    block_keys,
    indexer_topk_two_stage,
    two_stage_plan,
    indexer_merge_chunk,
    indexer_select_chunk,
    indexer_topk,
    materialize_scores,
    materialize_topk,
    plan,
    quantize_q,
    sparse_attention,
    workspace,
    workspace_bytes,
)
from ._lib import SiError  # noqa: F401

_lib.load()

__all__ = [
    "Plan", "TwoStagePlan", "block_keys", "indexer_topk_two_stage", "two_stage_plan", "SiError", "indexer_topk", "indexer_select_chunk", "indexer_merge_chunk",
    "materialize_scores", "materialize_topk", "plan", "quantize_q", "sparse_attention", "workspace", "workspace_bytes",
]
