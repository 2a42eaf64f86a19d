"""Pins of the sparse-attention oracle against closed forms: equal logits give the
mean of the selected values, two entries give the logistic weights, one dominant
entry gives its value, padding and order do not matter, an empty selection gives
zeros.  Planted slips (no max subtraction is harmless; a wrong scale, the weights not
normalised, padding read as key 0) must each fail a pin."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as OA
from hand import bits

D = 128


def _bf(x):
    return bits(torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def test_equal_logits_give_the_mean():
    rnd = np.random.default_rng(1)
    kv = rnd.standard_normal((1, 9, D)).astype(np.float32)
    qa = np.zeros((1, 1, 3, D), dtype=np.float32)               # every logit 0
    idx = np.array([[[4, 0, 7, 2, -1, -1]]])
    o = oracle.sparse_attention(_bf(qa), _bf(kv), idx, 0.3)
    kvd = oracle.bf16_bits_to_f64(_bf(kv))
    want = kvd[0, [4, 0, 7, 2]].mean(axis=0)
    assert np.allclose(o[0, 0], want[None, :], rtol=0, atol=1e-15)


def test_two_entries_give_logistic_weights():
    """Keys e_0 * a and e_0 * b with q = e_0 * c: logits scale*c*a and scale*c*b, so
    the weight of the first is 1 / (1 + exp(scale c (b - a)))."""
    kv = np.zeros((1, 2, D), dtype=np.float32)
    kv[0, 0, 0], kv[0, 1, 0] = 1.5, -0.5
    kv[0, 0, 5], kv[0, 1, 5] = 2.0, 4.0
    qa = np.zeros((1, 1, 1, D), dtype=np.float32)
    qa[0, 0, 0, 0] = 3.0
    scale = 0.25
    o = oracle.sparse_attention(_bf(qa), _bf(kv), np.array([[[1, 0]]]), scale)
    w0 = 1.0 / (1.0 + math.exp(scale * 3.0 * (-0.5 - 1.5)))
    assert abs(o[0, 0, 0, 0] - (w0 * 1.5 + (1 - w0) * -0.5)) < 1e-14
    assert abs(o[0, 0, 0, 5] - (w0 * 2.0 + (1 - w0) * 4.0)) < 1e-14


def test_dominant_entry_and_empty_row():
    kv = np.zeros((1, 3, D), dtype=np.float32)
    kv[0, :, 0] = [1.0, 50.0, 2.0]
    kv[0, :, 1] = [7.0, -3.0, 9.0]
    qa = np.zeros((1, 2, 1, D), dtype=np.float32)
    qa[0, :, 0, 0] = 4.0
    idx = np.array([[[0, 1, 2], [-1, -1, -1]]])
    o = oracle.sparse_attention(_bf(qa), _bf(kv), idx, 1.0)
    assert abs(o[0, 0, 0, 1] - (-3.0)) < 1e-60 + 1e-12
    assert (o[0, 1] == 0).all()


def test_order_and_padding_do_not_matter():
    rnd = np.random.default_rng(2)
    kv = rnd.standard_normal((1, 30, D)).astype(np.float32)
    qa = rnd.standard_normal((1, 1, 4, D)).astype(np.float32)
    sel = rnd.permutation(30)[:12]
    a = oracle.sparse_attention(_bf(qa), _bf(kv), np.concatenate([sel, [-1, -1]])[None, None], 0.09)
    b = oracle.sparse_attention(_bf(qa), _bf(kv), np.concatenate([sel[::-1], [-1] * 5])[None, None], 0.09)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_bound_is_reached_by_bf16_weight_rounding():
    """Two entries, values (1, 0) in dimension 0, logits 0 and ln(p0) with p0 just above
    1/2 so that its bf16 rounding loses almost 2^-8 of it: the output error of that
    rounding alone reaches half the bound (the other half is the output's own bf16
    rounding, of the same size).  A bound two times looser or tighter fails."""
    u8 = 2.0 ** -8
    p0 = 0.5 * (1 + u8 * (1 - 2 ** -6))              # rounds to 0.5 in bf16
    kv = np.zeros((1, 2, D), dtype=np.float32)
    kv[0, 0, 0] = 1.0
    # logit of entry 0 is scale * q . kv_0 = ln(p0) (q = 1, the scale carries the
    # logit); entry 1 has logit 0
    scale = math.log(p0)
    qa = np.zeros((1, 1, 1, D), dtype=np.float32)
    qa[0, 0, 0, 0] = 1.0
    qb = _bf(qa)
    p_exact = p0
    o = oracle.sparse_attention(qb, _bf(kv), np.array([[[0, 1]]]), scale)
    beta = oracle.attention_error_bound(qb, _bf(kv), np.array([[[0, 1]]]), scale)
    p_bf = float(torch.tensor(p_exact, dtype=torch.float32).to(torch.bfloat16))
    approx = p_bf / (p_exact + 1.0)                  # rounded numerator, exact denominator
    err = abs(approx - o[0, 0, 0, 0])
    assert err <= beta[0, 0, 0, 0]
    assert err >= 0.45 * beta[0, 0, 0, 0], err / beta[0, 0, 0, 0]


def _emulate_gpu(qa_bits, kv_bits, idx, scale):
    """fp32 / bf16 evaluation in the GPU's order of operations (fp32 logits times
    scale * log2(e), exp2 after the maximum, bf16-rounded weights in an fp32 weighted
    sum, fp32 sum of the unrounded weights, bf16 output)."""
    qa = oracle.bf16_bits_to_f64(qa_bits).astype(np.float32)
    kv = oracle.bf16_bits_to_f64(kv_bits).astype(np.float32)
    B, S, HA, _ = qa.shape
    sl2 = np.float32(scale * math.log2(math.e))
    out = np.zeros(qa.shape, dtype=np.float64)
    for b in range(B):
        for t in range(S):
            sel = idx[b, t][idx[b, t] >= 0]
            k = kv[b, sel]
            z = (qa[b, t] @ k.T).astype(np.float32) * sl2
            p = np.exp2(z - z.max(axis=1, keepdims=True)).astype(np.float32)
            pb = torch.from_numpy(p).to(torch.bfloat16).float().numpy()
            o = (pb @ k).astype(np.float32) * (np.float32(1) / p.sum(axis=1, dtype=np.float32))[:, None]
            out[b, t] = torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16).double().numpy()
    return out


@pytest.mark.parametrize("n,seed", [(4, 4), (8, 8), (512, 6)])
def test_bound_holds_and_is_reached_by_the_gpu_arithmetic(n, seed):
    """The emulated fp32/bf16 evaluation stays within the bound on random data; with
    few selected entries (where rounding errors of the weights do not average out) it
    reaches well over half of it (so a bound half as large fails)."""
    rnd = np.random.default_rng(seed)
    B, S, HA, T = 1, 24 if n < 64 else 6, 32, 700
    qa = _bf(rnd.standard_normal((B, S, HA, D)))
    kv = _bf(rnd.standard_normal((B, T, D)))
    idx = np.stack([rnd.permutation(T)[:n] for _ in range(S)])[None]
    scale = 1 / math.sqrt(D)
    o = oracle.sparse_attention(qa, kv, idx, scale)
    beta = oracle.attention_error_bound(qa, kv, idx, scale)
    err = np.abs(_emulate_gpu(qa, kv, idx, scale) - o)
    ratio = err / beta
    assert (ratio <= 1).all(), ratio.max()
    if n < 64:
        assert ratio.max() > 0.6, ratio.max()


@pytest.mark.parametrize("factor", [2.0, 0.5])
def test_bound_planted_scalings_are_caught(factor, monkeypatch):
    orig = OA.attention_error_bound
    monkeypatch.setattr(oracle, "attention_error_bound",
                        lambda *a, **k: orig(*a, **k) * factor)
    caught = 0
    for pin in (test_bound_is_reached_by_bf16_weight_rounding,
                lambda: test_bound_holds_and_is_reached_by_the_gpu_arithmetic(4, 4),
                lambda: test_bound_holds_and_is_reached_by_the_gpu_arithmetic(8, 8)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, factor


@pytest.mark.parametrize("mutant", ["wrong_scale", "not_normalised", "padding_as_key0"])
def test_attention_planted_mistakes_are_caught(mutant, monkeypatch):
    orig = OA.sparse_attention

    if mutant == "wrong_scale":
        def bad(qa_bits, kv_bits, idx, scale, rows=None):
            return orig(qa_bits, kv_bits, idx, scale * 2, rows=rows)
    elif mutant == "not_normalised":
        def bad(qa_bits, kv_bits, idx, scale, rows=None):
            out = orig(qa_bits, kv_bits, idx, scale, rows=rows)
            return out * 1.5
    else:
        def bad(qa_bits, kv_bits, idx, scale, rows=None):
            return orig(qa_bits, kv_bits, np.maximum(np.asarray(idx), 0), scale, rows=rows)
    monkeypatch.setattr(oracle, "sparse_attention", bad)
    caught = 0
    for pin in (test_equal_logits_give_the_mean, test_two_entries_give_logistic_weights,
                test_dominant_entry_and_empty_row, test_order_and_padding_do_not_matter):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, mutant
