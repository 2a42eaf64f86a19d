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

_DTYPE_NAMES = {"bf16": _lib.SI_BF16, "e4m3fn": _lib.SI_FP8_E4M3FN, "mxfp4": _lib.SI_MXFP4_E2M1}


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


def _q_dtype(q: torch.Tensor) -> int:
    """bf16 q, or E4M3 bytes (uint8 or float8_e4m3fn) from quantize_q."""
    if q.dtype == torch.bfloat16:
        return _lib.SI_BF16
    if q.dtype in (torch.uint8, torch.float8_e4m3fn):
        return _lib.SI_FP8_E4M3FN
    raise TypeError(f"q must be bfloat16 or E4M3 bytes (uint8), not {q.dtype}")


def _kc_dtype(kc: torch.Tensor, D: int, kc_dtype=None) -> int:
    """bf16 keys; uint8 keys of width D are E4M3 bytes, of width D/2 MXFP4 nibbles
    (or name the format: kc_dtype = "bf16" | "e4m3fn" | "mxfp4")."""
    if kc_dtype is not None:
        return _DTYPE_NAMES[kc_dtype]
    if kc.dtype == torch.bfloat16:
        return _lib.SI_BF16
    if kc.dtype == torch.float8_e4m3fn:
        return _lib.SI_FP8_E4M3FN
    if kc.dtype == torch.uint8:
        return _lib.SI_MXFP4_E2M1 if kc.shape[-1] * 2 == D else _lib.SI_FP8_E4M3FN
    raise TypeError(f"kc must be bfloat16, E4M3 bytes or MXFP4 bytes (uint8), not {kc.dtype}")


def _shapes(q, kc, w, kc_scale, kc_dtype=None):
    """Checks shapes, dtypes and placement; returns (B, S, T, H, D, q dtype, key dtype)."""
    if q.dim() != 4 or kc.dim() != 3 or w.dim() != 3:
        raise ValueError("expected q [B,S,H,D], kc [B,T,D] (MXFP4: [B,T,D/2]), w [B,S,H]")
    B, S, H, D = q.shape
    T = kc.shape[1]
    qd = _q_dtype(q)
    kd = _kc_dtype(kc, D, kc_dtype)
    width = D // 2 if kd == _lib.SI_MXFP4_E2M1 else D
    if kc.shape[0] != B or kc.shape[2] != width or tuple(w.shape) != (B, S, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kc {tuple(kc.shape)}, w {tuple(w.shape)}")
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    for name, t in (("q", q), ("kc", kc), ("w", w), ("kc_scale", kc_scale)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if kd == _lib.SI_FP8_E4M3FN and kc_scale is not None and (
            kc_scale.dtype != torch.float32 or tuple(kc_scale.shape) != (B, T)):
        raise ValueError("E4M3 keys: kc_scale must be float32 [B, T]")
    if kd == _lib.SI_MXFP4_E2M1 and kc_scale is not None and (
            kc_scale.dtype != torch.uint8 or tuple(kc_scale.shape) != (B, T, D // 32)):
        raise ValueError("MXFP4 keys: kc_scale must be uint8 E8M0 [B, T, D/32]")
    return B, S, T, H, D, qd, kd


_DTYPE_BY_CODE = {v: k for k, v in _DTYPE_NAMES.items()}


def plan(B, S, T, H=64, D=128, m=4, k=512, q_pos0=0, kc_dtype="bf16", key_tile=0,
         query_chunk=0, key_partition=0) -> Plan:
    """The driver's plan for a problem (host only, no device needed)."""
    lib = _lib.load()
    out = _lib.SiPlan()
    dt = _DTYPE_NAMES[kc_dtype]
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
                 out=None, ws=None, kc_dtype=None):
    """Top-k compressed keys per query row (streaming path).  Returns (idx int32
    [B,S,k], score float32 [B,S,k]) sorted by (score desc, idx asc), -1/-inf padded.
    q is bf16, or E4M3 bytes from quantize_q with w its effective weights."""
    B, S, T, H, D, qd, kcd = _shapes(q, kc, w, kc_scale, kc_dtype)
    pl = plan(B, S, T, H, D, m, k, q_pos0, _DTYPE_BY_CODE[kcd], key_tile, query_chunk,
              key_partition)
    if out is None:
        out = (torch.empty((B, S, k), dtype=torch.int32, device=q.device),
               torch.empty((B, S, k), dtype=torch.float32, device=q.device))
    if ws is None:
        ws = workspace(pl, q.device)
    cfg = _cfg(key_tile, query_chunk, key_partition)
    lib = _lib.load()
    _lib.check(lib.si_indexer_topk(
        _ptr(q), qd, _ptr(kc), kcd, _ptr(kc_scale), _ptr(w), B, S, T, H, D, m, k,
        q_pos0, ctypes.byref(cfg), _ptr(out[0]), _ptr(out[1]), _ptr(ws), ws.numel(),
        _stream(q.device)))
    return out


def indexer_select_chunk(q, kc, w, m, k, chunk, ws, *, kc_scale=None, q_pos0=0,
                         key_tile=0, query_chunk=0, key_partition=0, kc_dtype=None):
    """Select stage of one query chunk (fused scoring + local top-k into ws)."""
    B, S, T, H, D, qd, kcd = _shapes(q, kc, w, kc_scale, kc_dtype)
    cfg = _cfg(key_tile, query_chunk, key_partition)
    lib = _lib.load()
    _lib.check(lib.si_indexer_select_chunk(
        _ptr(q), qd, _ptr(kc), kcd, _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, k, q_pos0, ctypes.byref(cfg), chunk, _ptr(ws), ws.numel(), _stream(q.device)))


def indexer_merge_chunk(B, S, T, H, D, m, k, chunk, ws, out, *, q_pos0=0, kc_dtype="bf16",
                        key_tile=0, query_chunk=0, key_partition=0):
    """Merge stage of one query chunk (partition lists in ws -> rows of out)."""
    cfg = _cfg(key_tile, query_chunk, key_partition)
    dt = _DTYPE_NAMES[kc_dtype]
    lib = _lib.load()
    _lib.check(lib.si_indexer_merge_chunk(
        B, S, T, H, D, m, k, q_pos0, dt, ctypes.byref(cfg), chunk, _ptr(out[0]), _ptr(out[1]),
        _ptr(ws), ws.numel(), _stream(ws.device)))


def materialize_scores(q, kc, w, m, *, kc_scale=None, q_pos0=0, row0=0, rows=None, out=None,
                       kc_dtype=None):
    """Head-summed scores [B, rows, T] fp32 (-inf where masked), reference path."""
    B, S, T, H, D, qd, kcd = _shapes(q, kc, w, kc_scale, kc_dtype)
    rows = S - row0 if rows is None else rows
    if out is None:
        out = torch.empty((B, rows, T), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check(lib.si_materialize_scores(
        _ptr(q), qd, _ptr(kc), kcd, _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, q_pos0, row0, rows, _ptr(out), _stream(q.device)))
    return out


def materialize_topk(q, kc, w, m, k, *, kc_scale=None, q_pos0=0, row_block=None, out=None,
                     scores_ws=None, kc_dtype=None):
    """Materialise-then-select reference path; same output contract as indexer_topk."""
    B, S, T, H, D, qd, kcd = _shapes(q, kc, w, kc_scale, kc_dtype)
    row_block = max(1, min(S, 4096)) if row_block is None else row_block
    if out is None:
        out = (torch.empty((B, S, k), dtype=torch.int32, device=q.device),
               torch.empty((B, S, k), dtype=torch.float32, device=q.device))
    if scores_ws is None:
        scores_ws = torch.empty(max(1, B * min(row_block, max(S, 1)) * T), dtype=torch.float32,
                                device=q.device)
    lib = _lib.load()
    _lib.check(lib.si_materialize_topk(
        _ptr(q), qd, _ptr(kc), kcd, _ptr(kc_scale), _ptr(w), B, S, T, H, D,
        m, k, q_pos0, _ptr(out[0]), _ptr(out[1]), _ptr(scores_ws), scores_ws.numel() * 4,
        row_block, _stream(q.device)))
    return out


def quantize_q(q, w, *, out=None, with_scale=False):
    """si_quantize_q_e4m3: per-(row, head) E4M3 q and the effective weights w * scale.
    q bf16 [B, S, H, D], w float32 [B, S, H].  Returns (q8 uint8 [B, S, H, D], w_eff
    float32 [B, S, H]) and, with with_scale, the scales [B, S, H] as a third item."""
    if q.dim() != 4 or w.dim() != 3 or tuple(w.shape) != tuple(q.shape[:3]):
        raise ValueError("expected q [B,S,H,D] and w [B,S,H]")
    if q.dtype != torch.bfloat16 or w.dtype != torch.float32:
        raise TypeError("q must be bfloat16 and w float32")
    for name, t in (("q", q), ("w", w)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    B, S, H, D = q.shape
    if out is None:
        out = (torch.empty((B, S, H, D), dtype=torch.uint8, device=q.device),
               torch.empty((B, S, H), dtype=torch.float32, device=q.device))
    scale = torch.empty((B, S, H), dtype=torch.float32, device=q.device) if with_scale else None
    lib = _lib.load()
    _lib.check(lib.si_quantize_q_e4m3(_ptr(q), _ptr(w), B * S, H, D, _ptr(out[0]), _ptr(out[1]),
                                      _ptr(scale), _stream(q.device)))
    return (*out, scale) if with_scale else out


# ---- two-stage (coarse -> fine) indexer ----------------------------------------------

def block_keys(kc, block: int = 8, out=None):
    """si_block_keys_mean: bf16 block keys [B, T // block, D] (bf16-rounded mean of each
    block of `block` consecutive keys, fp32 sum in key order)."""
    if kc.dim() != 3 or kc.dtype != torch.bfloat16 or not kc.is_cuda or not kc.is_contiguous():
        raise ValueError("kc must be a contiguous bf16 GPU tensor [B, T, D]")
    B, T, D = kc.shape
    if out is None:
        out = torch.empty((B, T // block, D), dtype=torch.bfloat16, device=kc.device)
    lib = _lib.load()
    _lib.check(lib.si_block_keys_mean(_ptr(kc), _lib.SI_BF16, B, T, D, block, _ptr(out),
                                      _stream(kc.device)))
    return out


@dataclass(frozen=True)
class TwoStagePlan:
    query_chunk: int
    n_chunks: int
    cand_stride: int
    workspace_bytes: int


def two_stage_plan(B, S, T, H=64, D=128, m=4, k=512, k_blocks=2048, block=8, q_pos0=0,
                   query_chunk=0, key_tile=0, key_partition=0) -> TwoStagePlan:
    lib = _lib.load()
    out = _lib.SiTwoStagePlan()
    cfg = _cfg(key_tile, query_chunk, key_partition)
    _lib.check(lib.si_indexer_two_stage_plan(B, S, T, H, D, m, k, k_blocks, block, q_pos0,
                                             ctypes.byref(cfg), ctypes.byref(out)))
    return TwoStagePlan(out.query_chunk, out.n_chunks, out.cand_stride, out.workspace_bytes)


def indexer_topk_two_stage(q, kc, kb, w, m: int, k: int, *, k_blocks: int = 2048,
                           block: int = 8, q_pos0: int = 0, query_chunk: int = 0,
                           key_tile: int = 0, key_partition: int = 0, out=None, ws=None):
    """Two-stage top-k (coarse blocks, then fine keys).  kb = block_keys(kc, block).
    Returns (idx int32 [B,S,k], score float32 [B,S,k]) like indexer_topk."""
    B, S, T, H, D, qd, kcd = _shapes(q, kc, w, None)
    if qd != _lib.SI_BF16 or kcd != _lib.SI_BF16:
        raise TypeError("the two-stage indexer takes bf16 q and bf16 keys")
    if tuple(kb.shape) != (B, T // block, D) or kb.dtype != torch.bfloat16 or not kb.is_contiguous():
        raise ValueError("kb must be the bf16 block keys [B, T // block, D]")
    pl = two_stage_plan(B, S, T, H, D, m, k, k_blocks, block, q_pos0, query_chunk, key_tile,
                        key_partition)
    if out is None:
        out = (torch.empty((B, S, k), dtype=torch.int32, device=q.device),
               torch.empty((B, S, k), dtype=torch.float32, device=q.device))
    if ws is None:
        ws = torch.empty(max(pl.workspace_bytes, 1), dtype=torch.uint8, device=q.device)
    cfg = _cfg(key_tile, query_chunk, key_partition)
    lib = _lib.load()
    _lib.check(lib.si_indexer_topk_two_stage(
        _ptr(q), qd, _ptr(kc), kcd, _ptr(kb), _ptr(w), B, S, T, H, D, m, k, k_blocks, block,
        q_pos0, ctypes.byref(cfg), _ptr(out[0]), _ptr(out[1]), _ptr(ws), ws.numel(),
        _stream(q.device)))
    return out


# ---- sparse-attention consumer ---------------------------------------------------------

def sparse_attention(qa, kv, idx, scale=None, *, out=None):
    """si_sparse_attention: softmax attention of qa [B, S, HA, D] over the selected
    compressed latents kv[b, idx[b, t, :]] (key = value), idx [B, S, k] int32 (-1 padded,
    e.g. indexer_topk's indices).  scale defaults to 1/sqrt(D).  Returns bf16
    [B, S, HA, D]."""
    if qa.dim() != 4 or kv.dim() != 3 or idx.dim() != 3:
        raise ValueError("expected qa [B,S,HA,D], kv [B,T,D], idx [B,S,k]")
    B, S, HA, D = qa.shape
    T = kv.shape[1]
    if kv.shape[0] != B or kv.shape[2] != D or tuple(idx.shape[:2]) != (B, S):
        raise ValueError("shape mismatch")
    if qa.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16 or idx.dtype != torch.int32:
        raise TypeError("qa and kv must be bfloat16, idx int32")
    for name, t in (("qa", qa), ("kv", kv), ("idx", idx)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    k = idx.shape[2]
    scale = 1.0 / (D ** 0.5) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, S, HA, D), dtype=torch.bfloat16, device=qa.device)
    lib = _lib.load()
    _lib.check(lib.si_sparse_attention(_ptr(qa), _ptr(kv), _ptr(idx), B, S, T, HA, D, k,
                                       ctypes.c_float(scale), _ptr(out), _stream(qa.device)))
    return out
