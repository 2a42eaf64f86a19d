"""Plain CPU oracle of the two-stage (coarse -> fine) indexer.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP product path shares no code with it.

The chengshu blog page "两级稀疏注意力：滑窗、压缩 KV latent 与 indexer", section
"indexer：在摘要里做'预筛选'", describes the indexer of a later model as two stages:
a cheap candidate stage that scores blocks of 8 compressed latents and keeps 2048
blocks, then fine scoring of the candidates that keeps the best 512 latents.  The
page does not define a block's score.  Readings adopted (each the plainest one the
page supports):

* A block's key is the element-wise mean of its 8 compressed keys: summed in fp32 in
  key order, multiplied by 1/8 (exact), rounded to bf16 (nearest, ties to even).  Its
  score is the indexer score of that key (the same formula as a compressed key's), so
  the coarse stage is the single-stage indexer over block keys.
* Block j (keys 8j .. 8j+7) is a candidate for query t only when all of its keys are
  visible: (8j + 8) m <= t + 1, i.e. the causal mask with ratio 8m.  The coarse stage
  keeps the top min(2048, complete blocks) blocks by (score desc, block index asc).
* The fine candidates are every key of the kept blocks plus the visible keys of the
  query's trailing incomplete block (at most 7), so no visible key is left out because
  its block is not complete yet; the fine stage keeps the top-k of those by
  (score desc, key index asc), padded with -1 / -inf.
So whenever a query sees at most 2048 complete blocks, every visible key is a fine
candidate and the result is the single-stage top-k.
"""

from __future__ import annotations

import numpy as np

from .indexer import _decode_q, bf16_bits_to_f64, score_row, select_topk, visible_count


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """bf16 bit patterns of fp32 values: round to nearest, ties to the even bf16 (finite
    inputs).  Written from the definition: the kept 16 bits are rounded up when the
    dropped 16 bits exceed half, or equal half and the kept value is odd."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    drop = u & np.uint64(0xFFFF)
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & np.uint64(1)) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def block_keys_mean(kc_bits, block: int = 8) -> np.ndarray:
    """Block keys [B, T // block, D] as bf16 bits from bf16 keys [B, T, D]: the fp32 sum
    k_{bj} + k_{bj+1} + ... in key order, times 1/block (block a power of two), rounded
    to bf16.  Keys past the last complete block have no block key."""
    kf = bf16_bits_to_f64(kc_bits).astype(np.float32)
    B, T, D = kf.shape
    nb = T // block
    acc = kf[:, 0:nb * block:block].copy()
    for i in range(1, block):
        acc = (acc + kf[:, i:nb * block:block]).astype(np.float32)
    mean = (acc * np.float32(1.0 / block)).astype(np.float32)
    return f32_to_bf16_bits_rne(mean)


def two_stage_topk(q_bits, kc_bits, w, m: int, k: int, *, k_blocks: int = 2048,
                   block: int = 8, q_pos0: int = 0, rows=None, q_dtype: str = "bf16",
                   return_candidates: bool = False):
    """Two-stage top-k for the query rows ``rows`` (default all) of every batch entry.

    q_bits [B, S, H, D], kc_bits [B, T, D] bf16 keys, w [B, S, H].  Returns idx int64
    [B, R, k] and score float64 [B, R, k] (and, with return_candidates, the list of
    candidate key arrays per (b, row))."""
    q_bits = np.asarray(q_bits)
    w = np.asarray(w, dtype=np.float32)
    B, S, H, D = q_bits.shape
    kd = bf16_bits_to_f64(kc_bits)
    T = kd.shape[1]
    bd = bf16_bits_to_f64(block_keys_mean(kc_bits, block))
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out_idx = np.full((B, rows.shape[0], k), -1, dtype=np.int64)
    out_val = np.full((B, rows.shape[0], k), -np.inf, dtype=np.float64)
    cands_all = []
    for b in range(B):
        for i, r in enumerate(rows):
            t = q_pos0 + int(r)
            n = visible_count(t, m, T)
            nb = visible_count(t, block * m, T // block)      # complete visible blocks
            qd = _decode_q(q_bits[b, r], q_dtype)
            wd = w[b, r].astype(np.float64)
            if nb > 0:
                bs = score_row(qd, wd, bd[b, :nb], np.ones(nb))
                sel, _ = select_topk(bs, min(k_blocks, nb))
                blocks = np.sort(sel[sel >= 0])
            else:
                blocks = np.zeros(0, dtype=np.int64)
            cand = (block * blocks[:, None] + np.arange(block)[None, :]).reshape(-1)
            cand = np.concatenate([cand, np.arange(block * nb, n)]).astype(np.int64)
            cands_all.append(cand)
            if cand.size == 0:
                continue
            sc = score_row(qd, wd, kd[b, cand], np.ones(cand.size))
            order = np.lexsort((cand, -sc))[:k]
            out_idx[b, i, :order.size] = cand[order]
            out_val[b, i, :order.size] = sc[order]
    if return_candidates:
        return out_idx, out_val, cands_all
    return out_idx, out_val
