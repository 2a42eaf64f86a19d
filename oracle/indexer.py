"""Plain CPU oracle of the CSA lightning-indexer top-k step.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP product path never calls it, links it
or shares code with it; the two meet only through the seeded inputs in ``synth/``.

What is computed (all in float64, inputs decoded from their raw bits by this
module's own decoders):

* StreamIndex abstract (quoted on the aisoku.com page "StreamIndex：ストリーミング
  Top-kによるメモリ制限付き圧縮スパースアテンション", Abstract): the lightning indexer
  scores the compressed keys and the top-k keys are kept per query; public
  implementations build the full ``[B, S, H_I, T]`` FP32 score tensor and then reduce
  it to top-k.  The oracle is that materialise-then-select definition, one query row
  at a time (it never needs the whole tensor, only one row of it).
* The pages describe the indexer only as a learned scoring projection over the
  compressed keys and print no formula.  Reading adopted: the DeepSeek lightning-indexer score
  ``I[t, s] = sum_h w[t, h] * max(0, sum_d q[t, h, d] * k[s, d])`` (no 1/sqrt(D), no
  softmax, ReLU before the head weighting).
* Causal mask (not on the pages; reading adopted): compressed key ``s`` is visible to
  query ``t`` iff ``(s + 1) * m <= t + 1``, with ``t`` the absolute query position.
  So ``n_t = min(T, (t + 1) // m)`` keys are visible and they are ``0 .. n_t - 1``.
* Tie-break (not on the pages; reading adopted): equal scores are ordered by lower key
  index first.  With it the top-k is unique.  Output rows are sorted by
  (score descending, index ascending); slots past ``min(k, n_t)`` hold index -1 and
  score -inf.
* fp8 keys (reading adopted): the per-row fp32 scale multiplies the per-head dot
  product before the ReLU.  Because the scale is positive this equals scaling after
  the ReLU or after the head sum, in exact arithmetic.

Every function here has at least one pin in ``tests/test_oracle_pins.py`` that does
not re-derive it from itself (hand-built cases, exact rational brute force, library
special cases, closed forms, exhaustive decoder tables).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats, decoded from raw bits.
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16/int16 array) to float64.

    bfloat16 is the upper half of an IEEE-754 binary32: the 16 bits shifted left by
    16 are the binary32 encoding of the same value, so the decode is exact.
    """
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3fn_value(b: int) -> float:
    """Value of one OCP FP8 E4M3 ('fn': finite, no infinities) byte.

    OCP 8-bit floating point specification: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^(1-7); S.1111.111 is
    NaN and there is no infinity, so the largest finite value is 1.75 * 2^8 = 448.
    """
    sign = -1.0 if (b & 0x80) else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 bytes (uint8/int8 array) to float64 through the table above."""
    return E4M3FN_TABLE[np.asarray(bits).astype(np.uint8)]


def _e2m1_value(c: int) -> float:
    """Value of one OCP FP4 E2M1 code (OCP Microscaling Formats specification): 1 sign
    bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 encodes the
    subnormal m/2 * 2^(1-1); no infinities or NaN, so the largest value is 1.5 * 2^2."""
    sign = -1.0 if (c & 0x8) else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return sign * (m / 2.0)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP MX E8M0 scale bytes: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(bits).astype(np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def mxfp4_bits_to_f64(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 rows: packed [..., D/2] bytes (element 2i in the low nibble of byte
    i, element 2i+1 in the high nibble) with one E8M0 scale per block of 32 elements,
    scales [..., D/32].  Value = E2M1(code) * 2^(scale - 127) (OCP MX: each block of 32
    elements shares one power-of-two scale)."""
    p = np.asarray(packed).astype(np.uint8)
    codes = np.stack([p & 0xF, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    v = E2M1_TABLE[codes]
    sc = np.repeat(e8m0_bits_to_f64(scales), 32, axis=-1)
    return v * sc


# ---------------------------------------------------------------------------
# Mask and counts.
# ---------------------------------------------------------------------------


def visible_count(t_abs: int, m: int, T: int) -> int:
    """Number of compressed keys visible to absolute query position ``t_abs``.

    Key s is visible iff (s + 1) * m <= t_abs + 1, so the visible keys are the prefix
    0 .. floor((t_abs + 1) / m) - 1, capped by the T keys that exist.
    """
    return max(0, min(T, (t_abs + 1) // m))


def total_visible_pairs(S: int, T: int, m: int, q_pos0: int = 0) -> int:
    """Sum over the S query rows of their visible-key counts (one batch entry)."""
    return sum(visible_count(q_pos0 + t, m, T) for t in range(S))


def materialized_score_bytes(B: int, S: int, H: int, T: int) -> int:
    """Bytes of the [B, S, H_I, T] FP32 per-head score tensor that public CSA
    implementations build before the top-k (StreamIndex abstract: 256 GB at
    S=65,536 with H_I=64 and m=4)."""
    return B * S * H * T * 4


# ---------------------------------------------------------------------------
# Scores and selection.
# ---------------------------------------------------------------------------


def _decode_keys(kc_bits, kc_dtype, kc_scale):
    """Keys as float64 [B, T, D] and the per-row scale [B, T] (ones for bf16 and for
    MXFP4, whose block scales are part of the decoded value)."""
    if kc_dtype == "bf16":
        kd = bf16_bits_to_f64(kc_bits)
        scale = np.ones(kd.shape[:2], dtype=np.float64)
    elif kc_dtype == "e4m3fn":
        kd = e4m3fn_bits_to_f64(kc_bits)
        if kc_scale is None:
            raise ValueError("fp8 keys need a per-row scale")
        scale = np.asarray(kc_scale, dtype=np.float32).astype(np.float64)
    elif kc_dtype == "mxfp4":
        if kc_scale is None:
            raise ValueError("MXFP4 keys need their E8M0 block scales")
        kd = mxfp4_bits_to_f64(kc_bits, kc_scale)
        scale = np.ones(kd.shape[:2], dtype=np.float64)
    else:
        raise ValueError(f"unknown key dtype {kc_dtype!r}")
    return kd, scale


def _decode_q(q_bits, q_dtype):
    """Query rows as float64: bf16 bit patterns, or E4M3 bytes (quantised q, whose
    scale the caller has folded into the head weights)."""
    if q_dtype == "bf16":
        return bf16_bits_to_f64(q_bits)
    if q_dtype == "e4m3fn":
        return e4m3fn_bits_to_f64(q_bits)
    raise ValueError(f"unknown q dtype {q_dtype!r}")


def score_row(q_row: np.ndarray, w_row: np.ndarray, keys: np.ndarray,
              scale: np.ndarray) -> np.ndarray:
    """Indexer scores of one query against the given keys, in float64.

    q_row [H, D] and keys [n, D] are already decoded, w_row is [H], scale is [n].
    z[h, s] = scale[s] * sum_d q[h, d] * k[s, d]; score[s] = sum_h w[h] * max(0, z[h, s]).
    """
    z = (q_row @ keys.T) * scale[None, :]
    return w_row @ np.maximum(z, 0.0)


def select_topk(scores: np.ndarray, k: int):
    """Top-k of one score row: stable order by (score descending, index ascending).

    Returns (idx int64 [k], score float64 [k]); slots past len(scores) are -1 / -inf.
    """
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))  # last key is primary
    keep = order[: min(k, n)]
    idx = np.full(k, -1, dtype=np.int64)
    val = np.full(k, -np.inf, dtype=np.float64)
    idx[: keep.shape[0]] = keep
    val[: keep.shape[0]] = scores[keep]
    return idx, val


def indexer_topk(q_bits, kc_bits, w, m: int, k: int, *, kc_dtype: str = "bf16",
                 kc_scale=None, q_pos0: int = 0, rows=None, q_dtype: str = "bf16"):
    """Oracle top-k for the query rows ``rows`` (default: all) of every batch entry.

    q_bits [B, S, H, D] bf16 bits (q_dtype "bf16") or E4M3 bytes ("e4m3fn", with w the
    effective weights w * q_scale); kc_bits [B, T, D] bf16 bits or E4M3 bytes, or
    [B, T, D/2] MXFP4 nibbles; w [B, S, H] float32; kc_scale [B, T] float32 for E4M3
    keys, [B, T, D/32] E8M0 bytes for MXFP4 keys.  Row r of q is the absolute query
    position q_pos0 + r.  Returns idx int64 [B, R, k] and score float64 [B, R, k] for
    the R requested rows.
    """
    q_bits = np.asarray(q_bits)
    w = np.asarray(w, dtype=np.float32)
    B, S, H, D = q_bits.shape
    kd, scale = _decode_keys(kc_bits, kc_dtype, kc_scale)
    T = kd.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out_idx = np.full((B, rows.shape[0], k), -1, dtype=np.int64)
    out_val = np.full((B, rows.shape[0], k), -np.inf, dtype=np.float64)
    for b in range(B):
        for i, r in enumerate(rows):
            n = visible_count(q_pos0 + int(r), m, T)
            if n == 0:
                continue
            qd = _decode_q(q_bits[b, r], q_dtype)
            sc = score_row(qd, w[b, r].astype(np.float64), kd[b, :n], scale[b, :n])
            out_idx[b, i], out_val[b, i] = select_topk(sc, k)
    return out_idx, out_val


def score_rows(q_bits, kc_bits, w, m: int, *, kc_dtype: str = "bf16", kc_scale=None,
               q_pos0: int = 0, rows=None, b: int = 0, q_dtype: str = "bf16"):
    """Full score rows [R, T] of batch entry ``b`` in float64, -inf where masked.

    This is one [R, T] slice of the head-summed score tensor that the materialise
    path reduces to top-k.
    """
    q_bits = np.asarray(q_bits)
    w = np.asarray(w, dtype=np.float32)
    S = q_bits.shape[1]
    kd, scale = _decode_keys(kc_bits, kc_dtype, kc_scale)
    T = kd.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((rows.shape[0], T), -np.inf, dtype=np.float64)
    for i, r in enumerate(rows):
        n = visible_count(q_pos0 + int(r), m, T)
        if n == 0:
            continue
        qd = _decode_q(q_bits[b, r], q_dtype)
        out[i, :n] = score_row(qd, w[b, r].astype(np.float64), kd[b, :n], scale[b, :n])
    return out


def score_error_bound(q_bits, kc_bits, w, m: int, *, kc_dtype: str = "bf16",
                      kc_scale=None, q_pos0: int = 0, rows=None, b: int = 0,
                      q_dtype: str = "bf16"):
    """Forward-error bound of an FP32 evaluation of each score, [R, T] float64.

    Textbook bound for a recursive sum of n terms in precision u = 2^-24:
    |fl(sum) - sum| <= n u sum |terms| (first order).  The score is a D-term dot per
    head (bf16 products are exact in fp32), scaled by the key scale, clamped at zero,
    then an H-term weighted sum, so the combined bound is
    (D + H + 2) * 2^-24 * sum_h |w_h| * scale_s * sum_d |q_hd k_sd|.
    The same bound holds for E4M3 q (products of two E4M3 values, or of an E4M3 and an
    MXFP4 value with its power-of-two block scale, are exact in fp32 as well).
    """
    q_bits = np.asarray(q_bits)
    w = np.asarray(w, dtype=np.float32)
    S, H, D = q_bits.shape[1:]
    kd, scale = _decode_keys(kc_bits, kc_dtype, kc_scale)
    T = kd.shape[1]
    u = 2.0 ** -24
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], T), dtype=np.float64)
    for i, r in enumerate(rows):
        n = visible_count(q_pos0 + int(r), m, T)
        if n == 0:
            continue
        qd = np.abs(_decode_q(q_bits[b, r], q_dtype))
        za = (qd @ np.abs(kd[b, :n]).T) * scale[b, :n][None, :]
        out[i, :n] = (D + H + 2) * u * (np.abs(w[b, r].astype(np.float64)) @ za)
    return out
