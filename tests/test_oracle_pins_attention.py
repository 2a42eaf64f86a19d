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


def test_bound_covers_bf16_weight_rounding():
    """A weight set where every weight rounds in bf16 by almost 2^-9 relative: the
    output error of that rounding alone stays inside the bound."""
    kv = np.zeros((1, 2, D), dtype=np.float32)
    kv[0, 0, 0], kv[0, 1, 0] = 1.0, 0.0
    qa = np.zeros((1, 1, 1, D), dtype=np.float32)
    # logit difference so that exp2 of the smaller gives a value far from bf16's grid
    qa[0, 0, 0, 0] = -0.30078125
    o = oracle.sparse_attention(_bf(qa), _bf(kv), np.array([[[0, 1]]]), 1.0)
    beta = oracle.attention_error_bound(_bf(qa), _bf(kv), np.array([[[0, 1]]]), 1.0)
    p0 = math.exp(-0.30078125)
    p0_bf = float(torch.tensor(p0, dtype=torch.float32).to(torch.bfloat16))
    approx = p0_bf / (p0 + 1.0)                         # rounded numerator, exact denominator
    assert abs(approx - o[0, 0, 0, 0]) <= beta[0, 0, 0, 0]
    assert abs(approx - o[0, 0, 0, 0]) >= 0.05 * beta[0, 0, 0, 0]    # the bound is not loose


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
