"""Thin torch-facing binding of the C ABI: argument marshalling only.

Every step of the indexer runs in the HIP kernels of ``libsi_indexer.so``; torch only
supplies device memory (inputs, outputs and the workspace, so the caching allocator's
peak statistics see all of it) and the current stream.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

_KC_DTYPES = {torch.bfloat16: _lib.SI_BF16, torch.uint8: _lib.SI_FP8_E4M3FN,
              torch.float8_e4m3fn: _lib.SI_FP8_E4M3FN}


@dataclass(frozen=True)
class Plan:
    key_tile: int
    query_chunk: int
    key_partition: int
    n_partitions: int
    n_chunks: int
    cand_capacity: int
    workspace_bytes: int


def _cfg(key_tile=0, query_chunk=0, key_partition=0):
    return _lib.SiConfig(int(key_tile), int(query_chunk), int(key_partition), 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _kc_dtype(kc: torch.Tensor) -> int:
    try:
        return _KC_DTYPES[kc.dtype]
    except KeyError:
        raise TypeError(f"kc must be bfloat16 or E4M3 bytes (uint8), not {kc.dtype}") from None


def _shapes(q, kc, w, kc_scale):
    if q.dim() != 4 or kc.dim() != 3 or w.dim() != 3:
        raise ValueError("expected q [B,S,H,D], kc [B,T,D], w [B,S,H]")
    B, S, H, D = q.shape
    T = kc.shape[1]
    if kc.shape[0] != B or kc.shape[2] != D or tuple(w.shape) != (B, S, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kc {tuple(kc.shape)}, w {tuple(w.shape)}")
    if q.dtype != torch.bfloat16 or w.dtype != torch.float32:
        raise TypeError("q must be bfloat16 and w float32")
    _kc_dtype(kc)
    for name, t in (("q", q), ("kc", kc), ("w", w), ("kc_scale", kc_scale)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if kc_scale is not None and (kc_scale.dtype != torch.float32 or tuple(kc_scale.shape) != (B, T)):
        raise ValueError("kc_scale must be float32 [B, T]")
    return B, S, T, H, D


def plan(B, S, T, H=64, D=128, m=4, k=512, q_pos0=0, kc_dtype="bf16", key_tile=0,
         query_chunk=0, key_partition=0) -> Plan:
    """The driver's plan for a problem (host only, no device needed)."""
    lib = _lib.load()
    out = _lib.SiPlan()
    dt = _lib.SI_BF16 if kc_dtype == "bf16" else _lib.SI_FP8_E4M3FN
    cfg = _cfg(key_tile, query_chunk, key_partition)
    _lib.check(lib.si_indexer_plan(B, S, T, H, D, m, k, q_pos0, dt, ctypes.byref(cfg),
                                   ctypes.byref(out)))
    return Plan(out.key_tile, out.query_chunk, out.key_partition, out.n_partitions,
                out.n_chunks, out.cand_capacity, out.workspace_bytes)


def workspace_bytes(B, S, T, H=64, D=128, m=4, k=512, key_tile=0, query_chunk=0,
                    key_partition=0) -> int:
    """si_indexer_topk_workspace_bytes: workspace bytes for q_pos0 = 0 (host only)."""
    lib = _lib.load()
    cfg = _cfg(key_tile, query_chunk, key_partition)
    n = lib.si_indexer_topk_workspace_bytes(B, S, T, H, D, m, k, ctypes.byref(cfg))
    if n == ctypes.c_size_t(-1).value:
        raise _lib.SiError(_lib.SI_ERR_INVALID_ARG, lib.si_last_error().decode())
    return int(n)


def workspace(pl: Plan, device) -> torch.Tensor:
    """A workspace tensor (uint8) large enough for the plan."""
    return torch.empty(max(pl.workspace_bytes, 1), dtype=torch.uint8, device=device)


def indexer_topk(q, kc, w, m: int, k: int, *, kc_scale=None, q_pos0: int = 0,
                 key_tile: int = 0, query_chunk: int = 0, key_partition: int = 0,
                 out=None, ws=None):
    """Top-k compressed keys per query row (streaming path).  Returns (idx int32
    [B,S,k], score float32 [B,S,k]) sorted by (score desc, idx asc), -1/-inf padded."""
    B, S, T, H, D = _shapes(q, kc, w, kc_scale)
    kcd = _kc_dtype(kc)
    pl = plan(B, S, T, H, D, m, k, q_pos0, "bf16" if kcd == _lib.SI_BF16 else "e4m3fn",
              key_tile, query_chunk, key_partition)
    if out is None:
        out = (torch.empty((B, S, k), dtype=torch.int32, device=q.device),
               torch.empty((B, S, k), dtype=torch.float32, device=q.device))
    if ws is None:
        ws = workspace(pl, q.device)
    cfg = _cfg(key_tile, query_chunk, key_partition)
    lib = _lib.load()
    _lib.check(lib.si_indexer_topk(
        _ptr(q), _lib.SI_BF16, _ptr(kc), kcd, _ptr(kc_scale), _ptr(w), B, S, T, H, D, m, k,
        q_pos0, ctypes.byref(cfg), _ptr(out[0]), _ptr(out[1]), _ptr(ws), ws.numel(),
        _stream(q.device)))
    return out


def indexer_select_chunk(q, kc, w, m, k, chunk, ws, *, kc_scale=None, q_pos0=0,
                         key_tile=0, query_chunk=0, key_partition=0):
    """Select stage of one query chunk (fused scoring + local top-k into ws)."""
    B, S, T, H, D = _shapes(q, kc, w, kc_scale)
    cfg = _cfg(key_tile, query_chunk, key_partition)
    lib = _lib.load()
    _lib.check(lib.si_indexer_select_chunk(
        _ptr(q), _lib.SI_BF16, _ptr(kc), _kc_dtype(kc), _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, k, q_pos0, ctypes.byref(cfg), chunk, _ptr(ws), ws.numel(), _stream(q.device)))


def indexer_merge_chunk(B, S, T, H, D, m, k, chunk, ws, out, *, q_pos0=0, kc_dtype="bf16",
                        key_tile=0, query_chunk=0, key_partition=0):
    """Merge stage of one query chunk (partition lists in ws -> rows of out)."""
    cfg = _cfg(key_tile, query_chunk, key_partition)
    dt = _lib.SI_BF16 if kc_dtype == "bf16" else _lib.SI_FP8_E4M3FN
    lib = _lib.load()
    _lib.check(lib.si_indexer_merge_chunk(
        B, S, T, H, D, m, k, q_pos0, dt, ctypes.byref(cfg), chunk, _ptr(out[0]), _ptr(out[1]),
        _ptr(ws), ws.numel(), _stream(ws.device)))


def materialize_scores(q, kc, w, m, *, kc_scale=None, q_pos0=0, row0=0, rows=None, out=None):
    """Head-summed scores [B, rows, T] fp32 (-inf where masked), reference path."""
    B, S, T, H, D = _shapes(q, kc, w, kc_scale)
    rows = S - row0 if rows is None else rows
    if out is None:
        out = torch.empty((B, rows, T), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check(lib.si_materialize_scores(
        _ptr(q), _lib.SI_BF16, _ptr(kc), _kc_dtype(kc), _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, q_pos0, row0, rows, _ptr(out), _stream(q.device)))
    return out


def materialize_topk(q, kc, w, m, k, *, kc_scale=None, q_pos0=0, row_block=None, out=None,
                     scores_ws=None):
    """Materialise-then-select reference path; same output contract as indexer_topk."""
    B, S, T, H, D = _shapes(q, kc, w, kc_scale)
    row_block = max(1, min(S, 4096)) if row_block is None else row_block
    if out is None:
        out = (torch.empty((B, S, k), dtype=torch.int32, device=q.device),
               torch.empty((B, S, k), dtype=torch.float32, device=q.device))
    if scores_ws is None:
        scores_ws = torch.empty(max(1, B * min(row_block, max(S, 1)) * T), dtype=torch.float32,
                                device=q.device)
    lib = _lib.load()
    _lib.check(lib.si_materialize_topk(
        _ptr(q), _lib.SI_BF16, _ptr(kc), _kc_dtype(kc), _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, k, q_pos0, _ptr(out[0]), _ptr(out[1]), _ptr(scores_ws), scores_ws.numel() * 4,
        row_block, _stream(q.device)))
    return out
