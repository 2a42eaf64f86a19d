"""Pins of the oracle's low-precision operands: the E4M3 encoder, the per-(row, head)
q quantisation, scoring with E4M3 q, and MXFP4 (E2M1 + E8M0) key decoding.

Each pin comes from outside the oracle: the OCP formats' own definitions checked
exhaustively (every code round-trips, every midpoint rounds to even), torch's own
casts and decoders, hand cases with exact values, and exact rational brute force.
``test_lowp_planted_mistakes_are_caught`` plants plausible slips and checks that a pin
fails for each."""

from __future__ import annotations

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.indexer as OI
import oracle.quant as OQ
import synth
from hand import bits

# ---------------------------------------------------------------------------
# E4M3 encoder
# ---------------------------------------------------------------------------

FINITE_CODES = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_e4m3_encode_roundtrips_every_finite_code():
    vals = oracle.e4m3fn_bits_to_f64(np.array(FINITE_CODES, dtype=np.uint8))
    got = OQ.e4m3fn_encode_rne(vals.astype(np.float32))
    want = np.array(FINITE_CODES, dtype=np.uint8)
    # +0 and -0 keep their own codes
    assert (got == want).all()


def test_e4m3_encode_midpoints_round_to_even():
    """Between adjacent non-negative E4M3 values a < b: the midpoint (exact in fp32)
    goes to whichever code is even, and one fp32 ulp either side of it goes to the
    nearer value; the same mirrored for negative values."""
    pos = [c for c in range(0x7F)]
    vals = oracle.e4m3fn_bits_to_f64(np.array(pos, dtype=np.uint8))
    for i in range(len(pos) - 1):
        a, b = vals[i], vals[i + 1]
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2
        even = pos[i] if pos[i] % 2 == 0 else pos[i + 1]
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        for sgn, sbit in ((1, 0), (-1, 0x80)):
            got = OQ.e4m3fn_encode_rne(np.array([sgn * mid, sgn * below, sgn * above],
                                                dtype=np.float32))
            assert got.tolist() == [even | sbit, pos[i] | sbit, pos[i + 1] | sbit], (a, b)


def test_e4m3_encode_matches_torch_cast():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even inside the range;
    it must agree on every bf16 value in [-448, 448] and on random fp32 values."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(allbits)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)].astype(np.float32)
    rnd = np.random.default_rng(5)
    r = (rnd.standard_normal(1 << 20) * rnd.choice([1e-3, 1e-1, 1, 30, 200], 1 << 20))
    r = np.clip(r, -448, 448).astype(np.float32)
    for x in (v, r):
        mine = OQ.e4m3fn_encode_rne(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (mine == ref).all()


# ---------------------------------------------------------------------------
# q quantisation
# ---------------------------------------------------------------------------

def test_quantize_q_hand_case():
    """amax 3.5 gives scale 3.5 / 448 = 2^-7 exactly, so every element is divided
    exactly: 3.5 -> 448 (0x7E), 1 -> 128 (0x70), -2 -> -256 (0xF8), 0.5 -> 64 (0x68),
    0 -> 0x00; w_eff = w * 2^-7.  A zero head keeps scale 1 and all-zero bytes."""
    q = np.zeros((1, 1, 2, 128), dtype=np.float32)
    q[0, 0, 0, :5] = [3.5, 1.0, -2.0, 0.5, 0.0]
    qb = bits(torch.from_numpy(q).to(torch.bfloat16))
    w = np.array([[[1.5, -3.0]]], dtype=np.float32)
    q8, w_eff, scale = oracle.quantize_q_e4m3(qb, w)
    assert q8[0, 0, 0, :5].tolist() == [0x7E, 0x70, 0xF8, 0x68, 0x00]
    assert (q8[0, 0, 0, 5:] == 0).all() and (q8[0, 0, 1] == 0).all()
    assert scale[0, 0].tolist() == [2.0 ** -7, 1.0]
    assert w_eff[0, 0].tolist() == [1.5 * 2.0 ** -7, -3.0]


def test_quantize_q_max_maps_to_448_and_error_is_half_an_e4m3_ulp():
    """On random bf16 q: each row's largest magnitude maps to +-448, and every element
    dequantises (code * scale) to within half an E4M3 spacing of q (plus the fp32
    division's own rounding)."""
    rnd = np.random.default_rng(2)
    q = torch.from_numpy(rnd.standard_normal((3, 17, 5, 128)).astype(np.float32)).to(torch.bfloat16)
    qb = bits(q)
    q8, w_eff, scale = oracle.quantize_q_e4m3(qb, np.ones((3, 17, 5), dtype=np.float32))
    qf = q.double().numpy()
    amax_pos = np.abs(qf).argmax(axis=-1)
    top = np.take_along_axis(q8, amax_pos[..., None], axis=-1)[..., 0]
    assert ((top & 0x7F) == 0x7E).all()
    deq = oracle.e4m3fn_bits_to_f64(q8) * scale[..., None].astype(np.float64)
    x = np.abs(qf) / scale[..., None]
    # spacing of E4M3 at |x|: 2^(floor(log2 x) - 3) for normals (x >= 2^-6), 2^-9 below
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -6)))
    half_gap = np.ldexp(1.0, (e - 4).astype(int)) * scale[..., None]
    assert (np.abs(deq - qf) <= half_gap * (1 + 2.0 ** -20) + 1e-30).all()
    assert (w_eff == scale).all()


def _brute_force(qv, kv, kscale, wv, m, k):
    S, H, D = len(qv), len(qv[0]), len(qv[0][0])
    T = len(kv)
    out = []
    for t in range(S):
        vis = [s for s in range(T) if (s + 1) * m <= t + 1]
        sc = []
        for s in vis:
            tot = Fraction(0)
            for h in range(H):
                dot = sum((qv[t][h][d] * kv[s][d] for d in range(D)), Fraction(0))
                tot += wv[t][h] * max(kscale[s] * dot, Fraction(0))
            sc.append((-tot, s))
        sc.sort()
        out.append([(s, -negv) for negv, s in sc[:k]])
    return out


E4M3_VALUES = {c: Fraction(float(v)) for c, v in
               zip(FINITE_CODES, oracle.e4m3fn_bits_to_f64(np.array(FINITE_CODES, np.uint8)))}


@pytest.mark.parametrize("seed", range(4))
def test_fp8_q_scores_exact_brute_force(seed):
    """E4M3 q bytes against E4M3 keys with a row scale (powers of two and 1.5, so every
    value is exact): the oracle's scores and order equal exact rational arithmetic."""
    rnd = random.Random(seed)
    S, T, H, D, m, k = 9, 6, 3, 6, rnd.choice([1, 2]), rnd.choice([2, 5])
    codes = [c for c in FINITE_CODES if abs(E4M3_VALUES[c]) <= 8 and
             E4M3_VALUES[c] == 0 or (0.125 <= abs(E4M3_VALUES[c]) <= 8)]
    q8 = np.array([[[[rnd.choice(codes) for _ in range(D)] for _ in range(H)]
                    for _ in range(S)]], dtype=np.uint8)
    k8 = np.array([[[rnd.choice(codes) for _ in range(D)] for _ in range(T)]], dtype=np.uint8)
    ks = np.array([[rnd.choice([0.5, 1.0, 1.5, 2.0]) for _ in range(T)]], dtype=np.float32)
    w = np.array([[[rnd.choice([-1.0, -0.25, 0.5, 2.0]) for _ in range(H)] for _ in range(S)]],
                 dtype=np.float32)
    idx, val = oracle.indexer_topk(q8, k8, w, m, k, q_dtype="e4m3fn", kc_dtype="e4m3fn",
                                   kc_scale=ks)
    qv = [[[E4M3_VALUES[int(c)] for c in q8[0, t, h]] for h in range(H)] for t in range(S)]
    kv = [[E4M3_VALUES[int(c)] for c in k8[0, s]] for s in range(T)]
    ref = _brute_force(qv, kv, [Fraction(float(x)) for x in ks[0]],
                       [[Fraction(float(x)) for x in w[0, t]] for t in range(S)], m, k)
    for t in range(S):
        assert idx[0, t].tolist() == [s for s, _ in ref[t]] + [-1] * (k - len(ref[t]))
        assert val[0, t, :len(ref[t])].tolist() == [float(v) for _, v in ref[t]]


def test_quantised_pipeline_equals_scaled_scores():
    """Quantise q, score with (E4M3 q, w_eff): equal to scoring the dequantised q
    (code * scale) with the original w, up to the fp32 rounding of w_eff only."""
    spec = synth.InputSpec(B=1, S=64, T=16, H=4, D=128, m=4, k=8, seed=41, kc_dtype="e4m3fn")
    x = synth.make_inputs(spec)
    qb = bits(x["q"])
    q8, w_eff, scale = oracle.quantize_q_e4m3(qb, x["w"].numpy())
    kb, ks = x["kc"].numpy(), x["kc_scale"].numpy()
    a = oracle.score_rows(q8, kb, w_eff, 4, q_dtype="e4m3fn", kc_dtype="e4m3fn", kc_scale=ks)
    # dequantised q in float64, original weights: the same up to w_eff's rounding
    deq = oracle.e4m3fn_bits_to_f64(q8) * scale[..., None].astype(np.float64)
    kd = oracle.e4m3fn_bits_to_f64(kb)[0] * ks[0][:, None].astype(np.float64)
    for t in range(spec.S):
        n = oracle.visible_count(t, 4, spec.T)
        z = deq[0, t] @ kd[:n].T
        ref = x["w"][0, t].double().numpy() @ np.maximum(z, 0)
        tol = 2.0 ** -24 * (np.abs(x["w"][0, t].double().numpy()) @ np.abs(np.maximum(z, 0))) * 1.01
        assert (np.abs(a[t, :n] - ref) <= tol + 1e-300).all()


# ---------------------------------------------------------------------------
# MXFP4 keys
# ---------------------------------------------------------------------------

def test_e2m1_values_through_torch_e4m3():
    """Every E2M1 value is an E4M3 value with the same sign, exponent rebiased by +6
    (bias 1 -> 7) and the mantissa bit moved to the top of E4M3's three; the subnormal
    0.5 is 2^-1.  torch's own E4M3 decoder gives each expected value."""
    for c in range(16):
        s, e, mbit = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and mbit == 0:
            want = -0.0 if s else 0.0
        elif e == 0:
            e4 = (s << 7) | ((-1 + 7) << 3)                        # 0.5 = 2^-1
            want = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).item()
        else:
            e4 = (s << 7) | ((e - 1 + 7) << 3) | (mbit << 2)
            want = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).item()
        got = oracle.E2M1_TABLE[c]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_e8m0_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    mine = oracle.e8m0_bits_to_f64(b)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_mxfp4_packing_hand_case():
    """Byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0); block scale
    byte 128 = 2^1 doubles them; the second block (scale 126 = 2^-1) holds code 0xF
    (-6) -> -3."""
    packed = np.zeros((1, 1, 32), dtype=np.uint8)
    packed[0, 0, 0] = 0x21
    packed[0, 0, 16] = 0xF0          # element 33 (block 1) = code 0xF
    scales = np.array([[[128, 126]]], dtype=np.uint8)
    v = oracle.mxfp4_bits_to_f64(packed, scales)[0, 0]
    assert v[0] == 1.0 and v[1] == 2.0 and v[32] == 0.0 and v[33] == -3.0
    assert (np.delete(v, [0, 1, 33]) == 0).all()


def test_mxfp4_generator_roundtrips_representable_values():
    """The synthetic MXFP4 keys: values that are E2M1 x 2^k with the block's largest
    magnitude 6 * 2^k come back exactly."""
    rnd = np.random.default_rng(3)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = rnd.choice(mags, (2, 5, 64)) * rnd.choice([-1, 1], (2, 5, 64))
    x[..., 0] = 6.0
    x[..., 32] = -6.0
    x = x * (2.0 ** rnd.integers(-3, 4, (2, 5, 1)))
    packed, sc = synth.mxfp4_quantize(torch.from_numpy(x.astype(np.float32)))
    back = oracle.mxfp4_bits_to_f64(packed.numpy(), sc.numpy())
    assert (back == x).all()


@pytest.mark.parametrize("seed", range(3))
def test_mxfp4_scores_exact_brute_force(seed):
    rnd = random.Random(seed)
    S, T, H, D, m, k = 8, 5, 2, 64, 1, 3
    q8 = np.array([[[[rnd.choice([0x00, 0x38, 0x40, 0xB8, 0x30, 0x44]) for _ in range(D)]
                     for _ in range(H)] for _ in range(S)]], dtype=np.uint8)
    codes = np.array([[[rnd.randrange(16) for _ in range(D)] for _ in range(T)]], dtype=np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    sc = np.array([[[rnd.choice([125, 127, 129]) for _ in range(D // 32)] for _ in range(T)]],
                  dtype=np.uint8)
    w = np.array([[[rnd.choice([-1.0, 0.5, 2.0]) for _ in range(H)] for _ in range(S)]],
                 dtype=np.float32)
    idx, val = oracle.indexer_topk(q8, packed, w, m, k, q_dtype="e4m3fn", kc_dtype="mxfp4",
                                   kc_scale=sc)
    qv = [[[E4M3_VALUES[int(c)] for c in q8[0, t, h]] for h in range(H)] for t in range(S)]
    e2m1 = [Fraction(float(v)) for v in
            [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]]
    kv = [[e2m1[int(codes[0, s, d])] * Fraction(2) ** (int(sc[0, s, d // 32]) - 127)
           for d in range(D)] for s in range(T)]
    ref = _brute_force(qv, kv, [Fraction(1)] * T,
                       [[Fraction(float(x)) for x in w[0, t]] for t in range(S)], m, k)
    for t in range(S):
        assert idx[0, t].tolist() == [s for s, _ in ref[t]] + [-1] * (k - len(ref[t]))
        assert val[0, t, :len(ref[t])].tolist() == [float(v) for _, v in ref[t]]


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _run(pins):
    caught = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            caught += 1
    return caught


@pytest.mark.parametrize("mutant", ["max_240", "ties_away", "w_not_scaled", "e2m1_bias0",
                                    "nibbles_swapped", "e8m0_bias128"])
def test_lowp_planted_mistakes_are_caught(mutant, monkeypatch):
    if mutant == "max_240":
        monkeypatch.setattr(OQ, "E4M3_MAX", 240.0)
        pins = [test_quantize_q_hand_case, test_quantize_q_max_maps_to_448_and_error_is_half_an_e4m3_ulp]
    elif mutant == "ties_away":
        orig = OQ.e4m3fn_encode_rne

        def away(x):
            x = np.asarray(x, dtype=np.float32)
            nudged = np.nextafter(x, np.where(x >= 0, np.float32(1e9), np.float32(-1e9)))
            nudged = np.clip(nudged, -448, 448)
            return orig(nudged)
        monkeypatch.setattr(OQ, "e4m3fn_encode_rne", away)
        pins = [test_e4m3_encode_midpoints_round_to_even, test_e4m3_encode_matches_torch_cast]
    elif mutant == "w_not_scaled":
        orig = OQ.quantize_q_e4m3

        def no_fold(q_bits, w):
            q8, _, scale = orig(q_bits, w)
            return q8, np.asarray(w, dtype=np.float32), scale
        monkeypatch.setattr(oracle, "quantize_q_e4m3", no_fold)
        pins = [test_quantize_q_hand_case, test_quantize_q_max_maps_to_448_and_error_is_half_an_e4m3_ulp]
    elif mutant == "e2m1_bias0":
        t = np.array([(1 if c < 8 else -1) * (((c >> 1) & 3 and (1 + (c & 1) / 2) * 2.0 ** ((c >> 1) & 3))
                                              or (c & 1) / 2) for c in range(16)])
        monkeypatch.setattr(OI, "E2M1_TABLE", t)
        monkeypatch.setattr(oracle, "E2M1_TABLE", t)
        pins = [test_e2m1_values_through_torch_e4m3, test_mxfp4_packing_hand_case,
                test_mxfp4_generator_roundtrips_representable_values]
    elif mutant == "nibbles_swapped":
        orig = OI.mxfp4_bits_to_f64

        def swapped(packed, scales):
            p = np.asarray(packed).astype(np.uint8)
            return orig(((p & 0xF) << 4) | (p >> 4), scales)
        monkeypatch.setattr(OI, "mxfp4_bits_to_f64", swapped)
        monkeypatch.setattr(oracle, "mxfp4_bits_to_f64", swapped)
        pins = [test_mxfp4_packing_hand_case, test_mxfp4_generator_roundtrips_representable_values]
    elif mutant == "e8m0_bias128":
        def biased(b):
            b = np.asarray(b).astype(np.int64)
            return np.where(b == 255, np.nan, np.ldexp(1.0, b - 128))
        monkeypatch.setattr(OI, "e8m0_bits_to_f64", biased)
        monkeypatch.setattr(oracle, "e8m0_bits_to_f64", biased)
        pins = [test_e8m0_matches_torch, test_mxfp4_packing_hand_case]
    assert _run(pins) > 0, mutant
