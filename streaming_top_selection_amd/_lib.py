"""ctypes view of ``libsi_indexer.so`` (declarations mirror ``include/si_indexer.h``).

Loading fails loudly if the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsi_indexer.so")

SI_OK, SI_ERR_INVALID_ARG, SI_ERR_UNSUPPORTED, SI_ERR_WORKSPACE, SI_ERR_HIP = range(5)
SI_BF16, SI_FP8_E4M3FN, SI_MXFP4_E2M1 = 1, 2, 3
SI_NOALLOC_SCRATCH_BYTES = 256 << 20      # include/si_indexer.h


class SiConfig(ctypes.Structure):
    _fields_ = [("key_tile", ctypes.c_int32), ("query_chunk", ctypes.c_int32),
                ("key_partition", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SiPlan(ctypes.Structure):
    _fields_ = [("key_tile", ctypes.c_int32), ("query_chunk", ctypes.c_int32),
                ("key_partition", ctypes.c_int32), ("n_partitions", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("cand_capacity", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


class SiTwoStagePlan(ctypes.Structure):
    _fields_ = [("query_chunk", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("cand_stride", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_cfgp = ctypes.POINTER(SiConfig)

# name -> (restype, argtypes); the list of entry points include/si_indexer.h declares
SIGNATURES = {
    "si_abi_version": (_i32, []),
    "si_status_str": (ctypes.c_char_p, [_i32]),
    "si_last_error": (ctypes.c_char_p, []),
    "si_indexer_plan": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _cfgp,
                               ctypes.POINTER(SiPlan)]),
    "si_indexer_topk_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _cfgp]),
    "si_indexer_topk": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32,
                               _i32, _i64, _cfgp, _p, _p, _p, _sz, _p]),
    "si_indexer_topk_noalloc": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i32,
                                       _i32, _i32, _i64, _cfgp, _p, _p, _p]),
    "si_indexer_select_chunk": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i32,
                                       _i32, _i32, _i64, _cfgp, _i32, _p, _sz, _p]),
    "si_indexer_merge_chunk": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _cfgp,
                                      _i32, _p, _p, _p, _sz, _p]),
    "si_quantize_q_e4m3": (_i32, [_p, _p, _i64, _i32, _i32, _p, _p, _p, _p]),
    "si_sparse_attention": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_float,
                                   _p, _p]),
    "si_block_keys_mean": (_i32, [_p, _i32, _i64, _i64, _i32, _i32, _p, _p]),
    "si_indexer_two_stage_plan": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i64, _cfgp, ctypes.POINTER(SiTwoStagePlan)]),
    "si_indexer_topk_two_stage": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _i64, _cfgp, _p, _p, _p,
                                         _sz, _p]),
    "si_materialize_scores": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i32,
                                     _i32, _i64, _i64, _i64, _p, _p]),
    "si_materialize_topk": (_i32, [_p, _i32, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i32, _i32,
                                   _i32, _i64, _p, _p, _p, _sz, _i64, _p]),
}

_LIB = None


def load():
    """The loaded library with argtypes set; raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python streaming_top_selection_amd/build.py` "
                "(there is no non-HIP fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


class SiError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        lib = load()
        super().__init__(f"{lib.si_status_str(status).decode()}: {detail}")


def check(status: int):
    if status != SI_OK:
        raise SiError(status, load().si_last_error().decode())
