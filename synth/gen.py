"""Seeded synthetic inputs for the lightning-indexer top-k step.

This module holds no part of the method's arithmetic: it only draws tensors.  Both the
HIP path (through the tests and the bench) and the CPU oracle consume what it makes.

Shapes follow the V4-Flash indexer dimensions the pages use (H_I = 64 indexer heads,
compression ratio m = 4, so T = S / m compressed keys), head dim D = 128, with the
value distributions and structure listed in ``CONFIGS``.

Every tensor is drawn in blocks of ``BLOCK_ROWS`` rows from a torch generator seeded by
(seed, tensor id, batch entry, block), so any block can be regenerated on its own (the
oracle only ever needs a few sampled rows of a large configuration).  The torch CPU and
GPU generators produce different streams: a tensor is defined by its seed *and* the
device it was drawn on, and tests copy inputs between devices rather than redraw them.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

BLOCK_ROWS = 4096

# tensor ids used in the seed mix
_TID_Q, _TID_K, _TID_W, _TID_CQ, _TID_CK, _TID_DUP, _TID_ROWS, _TID_QA, _TID_KV = range(1, 10)


@dataclasses.dataclass(frozen=True)
class InputSpec:
    B: int
    S: int
    T: int
    H: int = 64
    D: int = 128
    m: int = 4
    k: int = 512
    seed: int = 0
    kc_dtype: str = "bf16"          # "bf16", "e4m3fn" (+ per-row fp32 scale) or "mxfp4"
    w_std: float = 1.0 / 8.0        # w ~ N(0, 1) * w_std
    channel_scale: Optional[tuple] = None   # (lo, hi): per-channel U(lo, hi) scales
    dup_frac: float = 0.0           # fraction of keys that copy an earlier key

    def replace(self, **kw) -> "InputSpec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny indexer: the oracle checks every row in seconds.
    "tiny": InputSpec(B=1, S=1024, T=256, k=64, seed=1),
    # Small exactness check: 5% of keys are exact copies of earlier keys (score ties).
    "small": InputSpec(B=2, S=8192, T=2048, k=512, seed=2, dup_frac=0.05),
    # V4-Flash indexer layer at S = 64K with per-channel scales on q and k.
    "v4flash": InputSpec(B=1, S=65536, T=16384, k=512, seed=3, channel_scale=(0.5, 2.0)),
    # Long-context design sweep at S = 256K.
    "long": InputSpec(B=1, S=262144, T=65536, k=512, seed=4),
    # Million-token capacity run with E4M3 keys and a per-row fp32 scale.
    "million": InputSpec(B=1, S=1048576, T=262144, k=512, seed=5, kc_dtype="e4m3fn"),
    # The million-token shape with bf16 keys (single-stage against two-stage indexer).
    "million-bf16": InputSpec(B=1, S=1048576, T=262144, k=512, seed=5),
    # The V4-Flash layer with low-precision keys (the fp8-q paths quantise q themselves).
    "v4flash-e4m3": InputSpec(B=1, S=65536, T=16384, k=512, seed=3, channel_scale=(0.5, 2.0),
                              kc_dtype="e4m3fn"),
    "v4flash-mxfp4": InputSpec(B=1, S=65536, T=16384, k=512, seed=3, channel_scale=(0.5, 2.0),
                               kc_dtype="mxfp4"),
}

# E2M1 rounding boundaries: midpoints between the magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def mxfp4_quantize(x: torch.Tensor):
    """OCP MX FP4 of float32 rows x [..., D] (D a multiple of 32), the recipe of the OCP
    Microscaling Formats specification: each block of 32 elements gets the shared scale
    2^(floor(log2(max |x|)) - 2) (2 = the largest E2M1 exponent), stored as the E8M0
    byte exponent + 127; each element is x / scale rounded to the nearest E2M1 value
    (ties to the even code), saturated at +-6.  Returns (packed uint8 [..., D/2],
    element 2i in the low nibble of byte i; scales uint8 [..., D/32])."""
    *lead, D = x.shape
    xb = x.reshape(*lead, D // 32, 32).to(torch.float32)
    amax = xb.abs().amax(dim=-1)
    _, e = torch.frexp(amax)                      # amax = f * 2^e, f in [0.5, 1)
    shared = torch.where(amax > 0, e - 1 - 2, torch.full_like(e, -127)).clamp(-127, 127)
    y = xb * torch.pow(2.0, -shared.to(torch.float32))[..., None]     # exact power of 2
    a = y.abs().clamp(max=6.0)
    code = torch.zeros_like(a, dtype=torch.int32)
    for j, b in enumerate(_E2M1_MIDPOINTS):
        code += (a > b).to(torch.int32)
        if j % 2 == 1:                            # tie between codes j and j+1: take even j+1
            code += (a == b).to(torch.int32)
    code |= (torch.signbit(y).to(torch.int32) << 3)
    code = code.reshape(*lead, D).to(torch.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), (shared + 127).to(torch.uint8).contiguous()


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from a tuple of small integers (splitmix-style)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x ^= (p + 0x9E3779B97F4A7C15 + ((x << 6) & 0xFFFFFFFFFFFFFFFF) + (x >> 2))
        x &= 0xFFFFFFFFFFFFFFFF
        x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


def _randn_rows(spec, tid, b, r0, r1, inner, device):
    """Rows [r0, r1) of a [rows, *inner] N(0, 1) float32 tensor drawn block by block."""
    out = torch.empty((r1 - r0, *inner), dtype=torch.float32, device=device)
    blk = r0 // BLOCK_ROWS
    while blk * BLOCK_ROWS < r1:
        b0 = blk * BLOCK_ROWS
        g = _gen(device, spec.seed, tid, b, blk)
        x = torch.randn((BLOCK_ROWS, *inner), generator=g, dtype=torch.float32,
                        device=device)
        lo, hi = max(r0, b0), min(r1, b0 + BLOCK_ROWS)
        out[lo - r0:hi - r0] = x[lo - b0:hi - b0]
        blk += 1
    return out


def _channel_scales(spec, device):
    lo, hi = spec.channel_scale
    gq = _gen(device, spec.seed, _TID_CQ)
    gk = _gen(device, spec.seed, _TID_CK)
    cq = torch.rand(spec.D, generator=gq, device=device) * (hi - lo) + lo
    ck = torch.rand(spec.D, generator=gk, device=device) * (hi - lo) + lo
    return cq, ck


def gen_q_rows(spec: InputSpec, r0: int = 0, r1: Optional[int] = None, device="cpu"):
    """q rows [r0, r1) of every batch entry: bfloat16 [B, r1 - r0, H, D].

    Drawn and rounded one generator block at a time, so the float32 temporaries stay
    at one block (128 MiB at H = 64, D = 128) whatever the number of rows."""
    r1 = spec.S if r1 is None else r1
    out = torch.empty((spec.B, r1 - r0, spec.H, spec.D), dtype=torch.bfloat16, device=device)
    cq = _channel_scales(spec, device)[0] if spec.channel_scale else None
    for b in range(spec.B):
        lo = r0
        while lo < r1:
            hi = min(r1, (lo // BLOCK_ROWS + 1) * BLOCK_ROWS)
            x = _randn_rows(spec, _TID_Q, b, lo, hi, (spec.H, spec.D), device)
            if cq is not None:
                x = x * cq
            out[b, lo - r0:hi - r0] = x.to(torch.bfloat16)
            del x
            lo = hi
    return out


def gen_w_rows(spec: InputSpec, r0: int = 0, r1: Optional[int] = None, device="cpu"):
    """Head weights rows [r0, r1): float32 [B, r1 - r0, H], N(0, 1) * w_std."""
    r1 = spec.S if r1 is None else r1
    out = torch.empty((spec.B, r1 - r0, spec.H), dtype=torch.float32, device=device)
    for b in range(spec.B):
        out[b] = _randn_rows(spec, _TID_W, b, r0, r1, (spec.H,), device) * spec.w_std
    return out


def _duplicate_map(spec: InputSpec, b: int):
    """Source row for each key: identity except for floor(dup_frac * T) keys s >= 1,
    each of which copies a key s' < s that is itself not a copy (so the tie is visible
    whenever s is)."""
    T = spec.T
    src = torch.arange(T)
    n_dup = int(spec.dup_frac * T)
    if n_dup == 0 or T < 2:
        return src
    g = _gen("cpu", spec.seed, _TID_DUP, b)
    picked = torch.randperm(T - 1, generator=g)[:n_dup] + 1
    is_picked = torch.zeros(T, dtype=torch.bool)
    is_picked[picked] = True
    keep = torch.nonzero(~is_picked).flatten()           # sorted, contains 0
    picked, _ = torch.sort(picked)
    n_below = torch.searchsorted(keep, picked)           # keep positions < s
    u = torch.rand(n_dup, generator=g, dtype=torch.float64)
    choice = torch.minimum((u * n_below.to(torch.float64)).long(), n_below - 1)
    src[picked] = keep[choice]
    return src


def gen_keys(spec: InputSpec, device="cpu"):
    """Compressed keys for every batch entry.

    bf16 keys: (kc bfloat16 [B, T, D], None).
    mxfp4 keys: (kc uint8 [B, T, D/2] packed E2M1 codes, kc_scale uint8 [B, T, D/32]
    E8M0 block scales), see mxfp4_quantize.
    e4m3fn keys: (kc uint8 [B, T, D] holding OCP E4M3 bytes, kc_scale float32 [B, T]),
    where scale = max_d |x| / 448 and the byte is E4M3(round-to-nearest-even of
    clamp(x / scale, -448, 448)).  The clamp matters: torch's cast does not saturate.
    """
    ck = _channel_scales(spec, device)[1] if spec.channel_scale else None
    xs = []
    for b in range(spec.B):
        x = _randn_rows(spec, _TID_K, b, 0, spec.T, (spec.D,), device)
        if ck is not None:
            x = x * ck
        if spec.dup_frac > 0:
            x = x[_duplicate_map(spec, b).to(x.device)]
        xs.append(x)
    x = torch.stack(xs)
    if spec.kc_dtype == "bf16":
        return x.to(torch.bfloat16), None
    if spec.kc_dtype == "e4m3fn":
        scale = x.abs().amax(dim=-1) / 448.0
        scale = torch.where(scale > 0, scale, torch.ones_like(scale))
        y = torch.clamp(x / scale[..., None], -448.0, 448.0)
        return y.to(torch.float8_e4m3fn).view(torch.uint8), scale.to(torch.float32)
    if spec.kc_dtype == "mxfp4":
        return mxfp4_quantize(x)
    raise ValueError(f"unknown key dtype {spec.kc_dtype!r}")


def make_inputs(spec: InputSpec, device="cpu"):
    """All inputs of a configuration as a dict: q, kc, kc_scale (or None), w."""
    kc, kc_scale = gen_keys(spec, device)
    return {
        "q": gen_q_rows(spec, 0, spec.S, device),
        "kc": kc,
        "kc_scale": kc_scale,
        "w": gen_w_rows(spec, 0, spec.S, device),
    }


def duplicate_pairs(spec: InputSpec, b: int = 0):
    """(s, s') pairs of keys made identical by construction (s' < s)."""
    src = _duplicate_map(spec, b)
    s = torch.nonzero(src != torch.arange(spec.T)).flatten()
    return [(int(i), int(src[i])) for i in s]


def sample_rows(spec: InputSpec, n: int, salt: int = 100):
    """Sorted query rows to check against the oracle: n - 1 rows uniform over the rows
    that see at least k keys (t >= m * k - 1), plus the last row."""
    lo = min(spec.S - 1, spec.m * spec.k - 1)
    g = _gen("cpu", spec.seed + salt, _TID_ROWS)
    span = spec.S - lo
    pick = torch.randperm(span, generator=g)[: max(0, min(n - 1, span))] + lo
    rows = sorted(set(pick.tolist()) | {spec.S - 1})
    return rows


def gen_attention_inputs(spec: InputSpec, HA: int = 64, r0: int = 0, r1: Optional[int] = None,
                         device="cpu"):
    """Inputs of the sparse-attention consumer for query rows [r0, r1): attention queries
    qa bf16 [B, r1 - r0, HA, D] and the compressed latents kv bf16 [B, T, D] (key =
    value), both N(0, 1) rounded to bf16, drawn block by block like q."""
    r1 = spec.S if r1 is None else r1
    qa = torch.empty((spec.B, r1 - r0, HA, spec.D), dtype=torch.bfloat16, device=device)
    kv = torch.empty((spec.B, spec.T, spec.D), dtype=torch.bfloat16, device=device)
    for b in range(spec.B):
        lo = r0
        while lo < r1:
            hi = min(r1, (lo // BLOCK_ROWS + 1) * BLOCK_ROWS)
            qa[b, lo - r0:hi - r0] = _randn_rows(spec, _TID_QA, b, lo, hi, (HA, spec.D),
                                                 device).to(torch.bfloat16)
            lo = hi
        kv[b] = _randn_rows(spec, _TID_KV, b, 0, spec.T, (spec.D,), device).to(torch.bfloat16)
    return qa, kv
