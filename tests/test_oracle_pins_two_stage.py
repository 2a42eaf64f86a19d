"""Pins of the two-stage (coarse -> fine) indexer oracle.

From outside the oracle: torch's own fp32 -> bf16 cast, hand-built block keys, exact
rational brute force of the whole two-stage algorithm on inputs where every rounding
is exact, the reduction to the single-stage oracle when every complete block is
kept, and the candidate structure.  Planted slips must each fail a pin."""

from __future__ import annotations

import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.two_stage as OT
import synth
from hand import bits


def test_bf16_rounding_matches_torch():
    rnd = np.random.default_rng(1)
    x = (rnd.standard_normal(1 << 20) * 10.0 ** rnd.uniform(-30, 30, 1 << 20)).astype(np.float32)
    # exact midpoints between bf16 neighbours, and one fp32 ulp either side
    base = torch.from_numpy(rnd.standard_normal(4096).astype(np.float32)).to(torch.bfloat16)
    mid = (base.float().numpy().view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    for v in (x, mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))):
        mine = OT.f32_to_bf16_bits_rne(v)
        ref = torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (mine == ref).all()


def _bf16(vals):
    return bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


def test_block_keys_hand_cases():
    D = 128
    k = np.zeros((1, 17, D), dtype=np.float32)
    k[0, 0:8, 0] = 3.0                                   # equal keys: the mean is the key
    k[0, 0:8, 1] = [1, 2, 3, 4, 5, 6, 7, 8]              # 36 / 8 = 4.5
    k[0, 0:8, 2] = [1, 1, 1, 1, 1, 1, 1, 2.0 ** -3]      # 7.125 / 8 = 0.890625, exact in bf16
    # a mean exactly between two bf16 values: 1 + 2^-8 (midpoint of 1 and 1 + 2^-7)
    # rounds to the even 1.0; 1 + 3 * 2^-8 rounds up to the even 1 + 2^-6
    k[0, 8:16, 3] = [1 + 2.0 ** -8] * 8
    k[0, 8:16, 4] = [1 + 3 * 2.0 ** -8] * 8
    k[0, 16, 0] = 100.0                                  # the incomplete block: no key
    kb_in = bits(torch.from_numpy(k).to(torch.bfloat16))
    got = oracle.bf16_bits_to_f64(OT.block_keys_mean(kb_in, 8))
    assert got.shape == (1, 2, D)
    assert got[0, 0, 0] == 3.0 and got[0, 0, 1] == 4.5 and got[0, 0, 2] == 0.890625
    kin = oracle.bf16_bits_to_f64(kb_in)
    # the bf16 input values of block 1 (1 + 2^-8 is not bf16: the input rounds first)
    m3 = kin[0, 8:16, 3].mean()
    m4 = kin[0, 8:16, 4].mean()
    assert got[0, 1, 3] == m3 and got[0, 1, 4] == m4
    assert (got[0, 0, 5:] == 0).all()


def test_block_mean_rounding_ties_to_even():
    """Sums whose eighth lands exactly between two bf16 values (the key values are
    bf16; their fp32 sum is exact)."""
    D = 128
    k = np.zeros((1, 8, D), dtype=np.float32)
    # seven 1.0 and one 1 + 2^-7 * 8 * (odd half): mean = 1 + 2^-8 (tie -> 1.0), and
    # mean = 1 + 3*2^-8 (tie -> 1 + 2^-6)
    k[0, :, 0] = [1.0] * 7 + [1.0 + 8 * 2.0 ** -8]
    k[0, :, 1] = [1.0] * 7 + [1.0 + 8 * 3 * 2.0 ** -8]
    k[0, :, 2] = [1.0] * 7 + [1.0 + 8 * 5 * 2.0 ** -8]
    kin = torch.from_numpy(k).to(torch.bfloat16)
    assert torch.equal(kin.float(), torch.from_numpy(k))             # inputs exact in bf16
    got = oracle.bf16_bits_to_f64(OT.block_keys_mean(bits(kin), 8))[0, 0]
    assert got[0] == 1.0                        # 1 + 2^-8 -> even 1.0
    assert got[1] == 1.0 + 2.0 ** -6            # 1 + 3 * 2^-8 -> even 1 + 2^-6
    assert got[2] == 1.0 + 2 * 2.0 ** -7        # 1 + 2.5 * 2^-7 -> even 1 + 2 * 2^-7


def _brute_two_stage(qv, kv, wv, m, k, k_blocks, block):
    """Exact rational two-stage selection (Fraction arithmetic, exact block means)."""
    S, H, D = len(qv), len(qv[0]), len(qv[0][0])
    T = len(kv)

    def score(t, key):
        tot = Fraction(0)
        for h in range(H):
            dot = sum((qv[t][h][d] * key[d] for d in range(D)), Fraction(0))
            tot += wv[t][h] * max(dot, Fraction(0))
        return tot

    nbt = T // block
    bkeys = [[sum((kv[block * j + i][d] for i in range(block)), Fraction(0)) / block
              for d in range(D)] for j in range(nbt)]
    out = []
    for t in range(S):
        n = min(T, (t + 1) // m)
        nb = sum(1 for j in range(nbt) if (block * j + block) * m <= t + 1)
        bs = sorted(((-score(t, bkeys[j]), j) for j in range(nb)))[:k_blocks]
        cand = sorted([block * j + i for _, j in bs for i in range(block)] +
                      list(range(block * nb, n)))
        fs = sorted((-score(t, kv[s]), s) for s in cand)[:k]
        out.append([(s, -v) for v, s in fs])
    return out


@pytest.mark.parametrize("seed", range(5))
def test_two_stage_exact_brute_force(seed):
    """Keys and q in {-2..2}: block sums are integers below 17 in magnitude, so the fp32
    sum, the eighth and its bf16 rounding are exact, and every score is exact."""
    rnd = random.Random(seed)
    S, T, H, D, block = 40, 29, 2, 3, 4
    m = rnd.choice([1, 2])
    k, k_blocks = rnd.choice([(3, 2), (5, 3), (9, 2)])
    qv = [[[Fraction(rnd.randint(-2, 2)) for _ in range(D)] for _ in range(H)] for _ in range(S)]
    kv = [[Fraction(rnd.randint(-2, 2)) for _ in range(D)] for _ in range(T)]
    wv = [[Fraction(rnd.choice([-1, 1, 2])) for _ in range(H)] for _ in range(S)]
    q = torch.tensor([[[float(x) for x in h] for h in t] for t in qv])[None]
    kc = torch.tensor([[float(x) for x in s] for s in kv])[None]
    w = np.array([[[float(x) for x in t] for t in wv]], dtype=np.float32)
    # the oracle needs D = 128 nowhere: D is any size here
    idx, val = oracle.two_stage_topk(bits(q.to(torch.bfloat16)), bits(kc.to(torch.bfloat16)), w,
                                     m, k, k_blocks=k_blocks, block=block)
    ref = _brute_two_stage(qv, kv, wv, m, k, k_blocks, block)
    for t in range(S):
        want = [s for s, _ in ref[t]]
        assert idx[0, t, :len(want)].tolist() == want, (seed, t)
        assert (idx[0, t, len(want):] == -1).all()
        assert val[0, t, :len(want)].tolist() == [float(v) for _, v in ref[t]]


def test_two_stage_equals_single_stage_when_every_block_is_kept():
    spec = synth.InputSpec(B=2, S=300, T=75, H=4, m=4, k=16, seed=8)
    x = synth.make_inputs(spec)
    qb, kb, w = bits(x["q"]), bits(x["kc"]), x["w"].numpy()
    i1, v1 = oracle.two_stage_topk(qb, kb, w, 4, 16, k_blocks=10, block=8, q_pos0=3)
    i2, v2 = oracle.indexer_topk(qb, kb, w, 4, 16, q_pos0=3)
    assert (i1 == i2).all() and (v1 == v2).all()


def test_two_stage_candidates_structure():
    spec = synth.InputSpec(B=1, S=512, T=128, H=4, m=2, k=10, seed=9)
    x = synth.make_inputs(spec)
    kb_, qb, w = bits(x["kc"]), bits(x["q"]), x["w"].numpy()
    idx, _, cands = oracle.two_stage_topk(qb, kb_, w, 2, 10, k_blocks=3, block=8,
                                          return_candidates=True)
    for t in range(spec.S):
        n = oracle.visible_count(t, 2, spec.T)
        nb = oracle.visible_count(t, 16, spec.T // 8)       # complete visible blocks
        c = cands[t]
        assert len(c) == 8 * min(3, nb) + (n - 8 * nb)
        assert len(set(c.tolist())) == len(c) and (c < n).all()
        assert set(range(8 * nb, n)) <= set(c.tolist())          # the tail is always there
        got = [s for s in idx[0, t] if s >= 0]
        assert set(got) <= set(c.tolist()) and len(got) == min(10, len(c))


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


@pytest.mark.parametrize("mutant", ["any_key_visible", "no_tail", "coarse_ties_reversed",
                                    "sum_not_mean", "ties_away"])
def test_two_stage_planted_mistakes_are_caught(mutant, monkeypatch):
    pins = [lambda s=s: test_two_stage_exact_brute_force(s) for s in range(5)]
    pins += [test_two_stage_equals_single_stage_when_every_block_is_kept,
             test_two_stage_candidates_structure, test_block_keys_hand_cases,
             test_block_mean_rounding_ties_to_even, test_bf16_rounding_matches_torch]
    if mutant == "any_key_visible":
        orig = OT.visible_count

        def vis(t, m, T):          # a block counts once its first key is visible
            if T < 10 ** 6 and m % 8 == 0:
                return max(0, min(T, (t + 1 + m - m // 8) // m))
            return orig(t, m, T)
        monkeypatch.setattr(OT, "visible_count", vis)
    elif mutant == "no_tail":
        def no_tail(q_bits, kc_bits, w, m, k, *, k_blocks=2048, block=8, q_pos0=0, rows=None,
                    q_dtype="bf16", return_candidates=False):
            # the same two stages, but the trailing incomplete block's keys are dropped
            B, S = np.asarray(q_bits).shape[:2]
            kd = oracle.bf16_bits_to_f64(kc_bits)
            bd = oracle.bf16_bits_to_f64(OT.block_keys_mean(kc_bits, block))
            rows = np.arange(S) if rows is None else np.asarray(rows)
            idx = np.full((B, len(rows), k), -1, dtype=np.int64)
            val = np.full((B, len(rows), k), -np.inf)
            cands = []
            for b in range(B):
                for i, r in enumerate(rows):
                    nb = oracle.visible_count(q_pos0 + int(r), block * m, kd.shape[1] // block)
                    qd = oracle.bf16_bits_to_f64(q_bits[b, r])
                    wd = np.asarray(w[b, r], dtype=np.float64)
                    sel = oracle.select_topk(oracle.score_row(qd, wd, bd[b, :nb], np.ones(nb)),
                                             min(k_blocks, max(nb, 1)))[0] if nb else np.zeros(0, int)
                    sel = np.sort(sel[sel >= 0])
                    c = (block * sel[:, None] + np.arange(block)[None, :]).reshape(-1)
                    cands.append(c)
                    if c.size:
                        sc = oracle.score_row(qd, wd, kd[b, c], np.ones(c.size))
                        o = np.lexsort((c, -sc))[:k]
                        idx[b, i, :o.size], val[b, i, :o.size] = c[o], sc[o]
            return (idx, val, cands) if return_candidates else (idx, val)
        monkeypatch.setattr(oracle, "two_stage_topk", no_tail)
    elif mutant == "coarse_ties_reversed":
        def rev(scores, k):
            n = scores.shape[0]
            order = np.lexsort((-np.arange(n), -scores))
            keep = order[:min(k, n)]
            idx = np.full(k, -1, dtype=np.int64)
            v = np.full(k, -np.inf)
            idx[:keep.shape[0]] = keep
            v[:keep.shape[0]] = scores[keep]
            return idx, v
        monkeypatch.setattr(OT, "select_topk", rev)
    elif mutant == "sum_not_mean":
        orig = OT.block_keys_mean

        def summed(kc_bits, block=8):
            return OT.f32_to_bf16_bits_rne(oracle.bf16_bits_to_f64(orig(kc_bits, block)) * block)
        monkeypatch.setattr(OT, "block_keys_mean", summed)
    elif mutant == "ties_away":
        def away(x):
            u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
            return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)
        monkeypatch.setattr(OT, "f32_to_bf16_bits_rne", away)
    assert _run(pins) > 0, mutant
