"""Plain CPU oracle of the sparse-attention consumer.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP product path shares no code with it.

The pages compose the indexer with an attention kernel that reads only the selected
keys (StreamIndex abstract on the aisoku.com page, "a sparse attention kernel reads
only those", and the composition with a pipelined attention kernel at S = 262,144;
jeff.news page, sequence diagram: merge-topk passes the key indices to the sparse
attention, which reads only the selected keys).  The pages give no attention formula
or dimensions.  Reading adopted (the plainest one): for each query row t and attention
head h,
    o[t, h, :] = sum_j softmax_j(scale * <qa[t, h, :], kv[s_j, :]>) * kv[s_j, :]
over the selected compressed entries s_j of row t (the indexer's top-k, padding -1
excluded), with the compressed latent serving as both key and value, shared by all
heads (the MLA form of compressed sparse attention), scale = 1 / sqrt(D).  A row with
no selected entry outputs zeros.
"""

from __future__ import annotations

import math

import numpy as np

from .indexer import bf16_bits_to_f64


def sparse_attention(qa_bits, kv_bits, idx, scale: float, *, rows=None):
    """qa_bits [B, S, HA, D] bf16 bits, kv_bits [B, T, D] bf16 bits, idx [B, S, k]
    (-1 = none).  Returns o float64 [B, R, HA, D] for the rows `rows` (default all):
    softmax over the selected entries in float64, max-subtracted."""
    qa_bits = np.asarray(qa_bits)
    B, S, HA, D = qa_bits.shape
    kv = bf16_bits_to_f64(kv_bits)
    idx = np.asarray(idx)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, rows.shape[0], HA, D), dtype=np.float64)
    for b in range(B):
        for i, t in enumerate(rows):
            sel = idx[b, t][idx[b, t] >= 0]
            if sel.size == 0:
                continue
            q = bf16_bits_to_f64(qa_bits[b, t])                 # [HA, D]
            k = kv[b, sel]                                      # [n, D]
            logits = scale * (q @ k.T)                          # [HA, n]
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            out[b, i] = (p / p.sum(axis=1, keepdims=True)) @ k
    return out


def attention_error_bound(qa_bits, kv_bits, idx, scale: float, *, rows=None):
    """Element-wise bound [B, R, HA, D] on the error of the GPU evaluation: logits from
    bf16 products summed in fp32 and scaled, weights exp2 of fp32 logits rounded to
    bf16 for the weight x value product (fp32 accumulation), normalised by the fp32
    sum of the unrounded weights, output rounded to bf16.

    bf16 keeps 8 significant bits, so rounding to it changes a value by at most 2^-8
    of itself.  With w_j the exact weights and A_d = sum_j w_j |v_jd|, each computed
    weight is w_j (1 + e_j) with |e_j| <= eps_w = 2^-8 (its bf16 rounding) + 2 dz (the
    logit error dz in natural-log units, entering the weight and the maximum) + 2^-20
    (exp2 and the running-maximum rescales) + (n + 8) 2^-24 (the fp32 sums, the
    reciprocal and the final product), to first order, so before its own bf16 rounding
    the output is off by at most eps_w A_d (times 1 + 2^-6 for the second-order terms);
    that rounding adds 2^-8 of the output's magnitude:
        beta[d] = c eps_w A_d + 2^-8 (|o_d| + c eps_w A_d),   c = 1 + 2^-6.
    dz = (D + 4) 2^-24 |scale| max_j sum_d |qa_d kv_jd| (dot forward error, the scale
    products and the log2(e) factor)."""
    qa_bits = np.asarray(qa_bits)
    B, S, HA, D = qa_bits.shape
    kv = bf16_bits_to_f64(kv_bits)
    idx = np.asarray(idx)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    o = sparse_attention(qa_bits, kv_bits, idx, scale, rows=rows)
    out = np.zeros_like(o)
    u = 2.0 ** -24
    c = 1.0 + 2.0 ** -6
    for b in range(B):
        for i, t in enumerate(rows):
            sel = idx[b, t][idx[b, t] >= 0]
            n = sel.size
            if n == 0:
                continue
            q = bf16_bits_to_f64(qa_bits[b, t])
            k = kv[b, sel]
            logits = scale * (q @ k.T)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            w = p / p.sum(axis=1, keepdims=True)                # [HA, n]
            dz = (D + 4) * u * abs(scale) * (np.abs(q) @ np.abs(k).T).max(axis=1)   # [HA]
            eps_w = 2.0 ** -8 + 2 * dz + 2.0 ** -20 + (n + 8) * u
            A = w @ np.abs(k)                                   # [HA, D]
            e = c * eps_w[:, None] * A
            out[b, i] = e + 2.0 ** -8 * (np.abs(o[b, i]) + e)
    return out


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
