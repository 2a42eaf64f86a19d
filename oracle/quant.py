"""Plain CPU oracle of the indexer's low-precision operands.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; the HIP product path shares no code with it.

The pages name lower indexer precision as the other lever against the indexer's cost
(jeff.news "딥시크 V4 인덱서, 6기가바이트 메모리로…", 기술 맥락), and a deployment of the
same indexer that keeps its key cache in MXFP4 (chengshu blog "两级稀疏注意力：滑窗、
压缩 KV latent 与 indexer", section 部署视角).  They fix no quantisation scheme, so the
readings below are adopted (the per-token fp8 activation quantisation with a max-abs
scale that public DeepSeek indexer code uses for q):

* q is quantised per (query row, head): scale = max_d |q| / 448 in fp32 (448 is the
  largest finite OCP E4M3 value; scale 1 for an all-zero vector), each element is
  fp32(q / scale), clamped to [-448, 448], rounded to nearest E4M3 with ties to the
  even code.
* The scale is folded into the head weight: w_eff = fp32(w * scale).  Because the
  scale is positive, w * ReLU(scale * z) = (w * scale) * ReLU(z), so the scorer sees
  E4M3 q bytes and w_eff and never the scale itself.

Every decision that turns floating point into a code is taken in fp32, as on the GPU.
"""

from __future__ import annotations

import numpy as np

from .indexer import E4M3FN_TABLE, bf16_bits_to_f64

E4M3_MAX = 448.0

# the 127 non-negative finite E4M3 values in code order (codes 0x00 .. 0x7E), increasing
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def e4m3fn_encode_rne(x) -> np.ndarray:
    """OCP E4M3 code of each fp32 value |x| <= 448: the nearest E4M3 value, ties to the
    code with an even last mantissa bit (round to nearest even).  -0 keeps its sign
    bit.  Values beyond 448 are outside this function's domain (callers clamp)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3fn_encode_rne: |x| must be <= 448 and not NaN")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _POS_VALUES[lo], _POS_VALUES[hi]
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(a == vhi, _POS_CODES[hi], np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]))
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_q_e4m3(q_bits, w):
    """Per-(row, head) E4M3 quantisation of bf16 q with the scale folded into w.

    q_bits [..., H, D] bf16 bit patterns, w [..., H] fp32.  Returns (q8 uint8 [..., H, D],
    w_eff fp32 [..., H], scale fp32 [..., H]).  All arithmetic in fp32 (np.float32
    division and product, each correctly rounded)."""
    q = bf16_bits_to_f64(q_bits).astype(np.float32)          # exact: bf16 is a fp32 subset
    amax = np.abs(q).max(axis=-1)                              # exact
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    x = (q / scale[..., None]).astype(np.float32)
    x = np.clip(x, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    q8 = e4m3fn_encode_rne(x)
    w_eff = (np.asarray(w, dtype=np.float32) * scale).astype(np.float32)
    return q8, w_eff, scale
