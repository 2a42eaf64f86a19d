"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped ReLU, the weight
inside the ReLU, an off-by-one mask, a reversed tie-break, a transposed operand, a
wrong E4M3 exponent bias, a missing key scale) fails at least one of them;
``test_planted_mistakes_are_caught`` plants each slip and checks exactly that.
"""

from __future__ import annotations

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.indexer as OI
import synth
from hand import bits, build, expected, load_cases

CASES = load_cases()


# ---------------------------------------------------------------------------
# Hand-built cases (tests/golden/hand_cases.json)
# ---------------------------------------------------------------------------

def _run_hand(case):
    x = build(case)
    return oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), x["m"], x["k"],
                               kc_dtype=x["kc_dtype"],
                               kc_scale=None if x["kc_scale"] is None else x["kc_scale"].numpy(),
                               q_pos0=x["q_pos0"])


def _check_hand(case):
    idx, val = _run_hand(case)
    eidx, evals = expected(case)
    np.testing.assert_array_equal(idx, eidx, err_msg=case["name"])
    np.testing.assert_array_equal(val, evals, err_msg=case["name"])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case(case):
    _check_hand(case)


# ---------------------------------------------------------------------------
# Exact rational brute force on tiny random inputs (pure Python loops)
# ---------------------------------------------------------------------------

def _bf16_exact(v: float) -> Fraction:
    return Fraction(float(torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).float()))


def _brute_force(qv, kv, wv, m, k, q_pos0):
    """Exact scores with Fractions, exact ties, sort by (score desc, index asc)."""
    S, H, D = len(qv), len(qv[0]), len(qv[0][0])
    T = len(kv)
    out = []
    for t in range(S):
        vis = [s for s in range(T) if (s + 1) * m <= q_pos0 + t + 1]
        sc = []
        for s in vis:
            tot = Fraction(0)
            for h in range(H):
                dot = sum((qv[t][h][d] * kv[s][d] for d in range(D)), Fraction(0))
                tot += wv[t][h] * max(dot, Fraction(0))
            sc.append((-tot, s))
        sc.sort()
        row = [(s, -negv) for negv, s in sc[:k]]
        out.append(row)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_exact_brute_force(seed):
    rnd = random.Random(seed)
    S, T, H, D = 11, 6, 3, 5
    m = rnd.choice([1, 2, 3])
    k = rnd.choice([1, 2, 4, 7])
    q_pos0 = rnd.choice([0, 0, 3])
    # small dyadic values: every product and sum is exact in float64, and ties happen
    grid = [x / 2 for x in range(-6, 7)]
    qv = [[[Fraction(rnd.choice(grid)) for _ in range(D)] for _ in range(H)] for _ in range(S)]
    kv = [[Fraction(rnd.choice(grid)) for _ in range(D)] for _ in range(T)]
    wv = [[Fraction(rnd.choice([-2, -1, -0.5, 0.5, 1, 1.5])) for _ in range(H)] for _ in range(S)]
    q = torch.tensor([[[float(x) for x in row] for row in head] for head in qv])[None].to(torch.bfloat16)
    kc = torch.tensor([[float(x) for x in row] for row in kv])[None].to(torch.bfloat16)
    w = np.asarray([[float(x) for x in row] for row in wv], dtype=np.float32)[None]
    idx, val = oracle.indexer_topk(bits(q), bits(kc), w, m, k, q_pos0=q_pos0)
    ref = _brute_force(qv, kv, wv, m, k, q_pos0)
    for t in range(S):
        want_idx = [s for s, _ in ref[t]] + [-1] * (k - len(ref[t]))
        want_val = [float(v) for _, v in ref[t]] + [-math.inf] * (k - len(ref[t]))
        assert idx[0, t].tolist() == want_idx, (seed, t)
        assert val[0, t].tolist() == want_val, (seed, t)


def test_brute_force_with_bf16_rounded_values():
    """Random normal values (rounded to bf16 first): scores within 1e-12 relative of
    the exact rational result, and the same index sets wherever the gap between the
    k-th and (k+1)-th exact score is not tiny."""
    rnd = np.random.default_rng(7)
    S, T, H, D, m, k = 9, 8, 4, 16, 1, 3
    q = torch.from_numpy(rnd.standard_normal((1, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    kc = torch.from_numpy(rnd.standard_normal((1, T, D)).astype(np.float32)).to(torch.bfloat16)
    w = rnd.standard_normal((1, S, H)).astype(np.float32)
    qv = [[[Fraction(float(x)) for x in q[0, t, h].float()] for h in range(H)] for t in range(S)]
    kv = [[Fraction(float(x)) for x in kc[0, s].float()] for s in range(T)]
    wv = [[Fraction(float(x)) for x in w[0, t]] for t in range(S)]
    idx, val = oracle.indexer_topk(bits(q), bits(kc), w, m, k)
    ref = _brute_force(qv, kv, wv, m, k, 0)
    for t in range(S):
        for j, (s, v) in enumerate(ref[t]):
            assert idx[0, t, j] == s
            assert abs(val[0, t, j] - float(v)) <= 1e-12 * max(1.0, abs(float(v)))


# ---------------------------------------------------------------------------
# Special case that reduces to a library routine
# ---------------------------------------------------------------------------

def test_single_head_nonnegative_reduces_to_matmul_topk():
    """H = 1, w = 1 and non-negative q, k: ReLU is the identity and the score matrix is
    q @ k^T; torch.topk on the causally masked matrix gives the same selection."""
    rnd = np.random.default_rng(3)
    S, T, D, m, k = 64, 16, 128, 4, 5
    q = torch.from_numpy(np.abs(rnd.standard_normal((1, S, 1, D))).astype(np.float32)).to(torch.bfloat16)
    kc = torch.from_numpy(np.abs(rnd.standard_normal((1, T, D))).astype(np.float32)).to(torch.bfloat16)
    w = np.ones((1, S, 1), dtype=np.float32)
    idx, val = oracle.indexer_topk(bits(q), bits(kc), w, m, k)
    full = q[0, :, 0].double() @ kc[0].double().T                    # [S, T]
    t = torch.arange(S)[:, None]
    s = torch.arange(T)[None, :]
    full = full.masked_fill((s + 1) * m > t + 1, -math.inf)
    ref_val, ref_idx = torch.topk(full, k, dim=1)
    for r in range(S):
        n = min(T, (r + 1) // m)
        nk = min(k, n)
        assert idx[0, r, :nk].tolist() == ref_idx[r, :nk].tolist()
        np.testing.assert_allclose(val[0, r, :nk], ref_val[r, :nk].numpy(), rtol=1e-12)
        assert (idx[0, r, nk:] == -1).all() and np.isneginf(val[0, r, nk:]).all()


def test_large_k_is_full_stable_sort():
    """k >= n_t returns every visible key, sorted by (score desc, index asc)."""
    spec = synth.InputSpec(B=1, S=40, T=10, H=2, D=128, m=4, k=64, seed=11)
    x = synth.make_inputs(spec)
    idx, val = oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), 4, 64)
    rows = oracle.score_rows(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), 4)
    for t in range(spec.S):
        n = oracle.visible_count(t, 4, spec.T)
        order = sorted(range(n), key=lambda s: (-rows[t, s], s))
        assert idx[0, t, :n].tolist() == order
        assert (idx[0, t, n:] == -1).all()


# ---------------------------------------------------------------------------
# Number formats: exhaustive against torch's own casts
# ---------------------------------------------------------------------------

def test_bf16_decoder_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_bits_to_f64(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_e4m3fn_decoder_exhaustive():
    allbits = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_bits_to_f64(allbits)
    ref = torch.from_numpy(allbits).view(torch.float8_e4m3fn).double().numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    finite = mine[np.isfinite(mine)]
    assert np.nanmax(np.abs(finite)) == 448.0
    assert int(np.isnan(mine).sum()) == 2                      # S.1111.111 only
    # every finite E4M3 value is exact in bf16, so an exact up-conversion exists
    as_bf16 = torch.from_numpy(finite.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert (as_bf16 == finite).all()


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_materialized_tensor_is_256_gib_at_64k():
    """[B, S, H_I, T] fp32 at S = 65,536, H_I = 64, m = 4 (T = 16,384): 2^38 bytes, the
    256 GB intermediate of the StreamIndex abstract."""
    assert oracle.materialized_score_bytes(1, 65536, 64, 65536 // 4) == 2 ** 38


@pytest.mark.parametrize("name", ["tiny", "small", "v4flash", "long"])
def test_visible_pair_count_closed_form(name):
    """With S = m T and m = 4: sum_t min(T, floor((t+1)/m)) = m T (T-1)/2 + T = T(2T-1)."""
    spec = synth.CONFIGS[name]
    T = spec.T
    assert spec.S == spec.m * T
    assert oracle.total_visible_pairs(spec.S, T, spec.m) == T * (2 * T - 1)


def test_visible_count_boundaries():
    for m in (1, 2, 3, 4, 7):
        for t in range(40):
            n = oracle.visible_count(t, m, 1000)
            assert all((s + 1) * m <= t + 1 for s in range(n))
            assert (n + 1) * m > t + 1
    assert oracle.visible_count(10 ** 6, 4, 5) == 5


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def _small_inputs(seed=5, **kw):
    spec = synth.InputSpec(B=2, S=96, T=24, H=4, D=128, m=4, k=8, seed=seed, **kw)
    return spec, synth.make_inputs(spec)


def test_weight_scaling_doubles_scores_exactly():
    spec, x = _small_inputs()
    i1, v1 = oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), 4, 8)
    i2, v2 = oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), 2 * x["w"].numpy(), 4, 8)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(2 * v1, v2)


def test_rows_are_independent_and_offset_slices_agree():
    spec, x = _small_inputs()
    qb, kb, w = bits(x["q"]), bits(x["kc"]), x["w"].numpy()
    full_i, full_v = oracle.indexer_topk(qb, kb, w, 4, 8)
    sub_i, sub_v = oracle.indexer_topk(qb[:, 40:70], kb, w[:, 40:70], 4, 8, q_pos0=40)
    np.testing.assert_array_equal(full_i[:, 40:70], sub_i)
    np.testing.assert_array_equal(full_v[:, 40:70], sub_v)
    one_i, one_v = oracle.indexer_topk(qb[1:], kb[1:], w[1:], 4, 8, rows=[77])
    np.testing.assert_array_equal(full_i[1:, 77:78], one_i)


def test_keys_past_visible_range_do_not_matter():
    spec, x = _small_inputs()
    qb, kb, w = bits(x["q"]), bits(x["kc"]).copy(), x["w"].numpy()
    i1, v1 = oracle.indexer_topk(qb, kb, w, 4, 8, rows=range(0, 40))
    kb[:, 10:] = 0x7F7F                                   # huge keys past row 39's view
    i2, v2 = oracle.indexer_topk(qb, kb, w, 4, 8, rows=range(0, 40))
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(v1, v2)


def test_duplicate_keys_tie_exactly_and_lower_index_wins():
    spec = synth.CONFIGS["small"].replace(S=2048, T=512, H=8, k=64)
    x = synth.make_inputs(spec)
    pairs = synth.duplicate_pairs(spec, 0)
    assert pairs
    rows = oracle.score_rows(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), 4, rows=[2047])
    for s, src in pairs:
        assert rows[0, s] == rows[0, src]
    idx, _ = oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), 4, 64, rows=[2047])
    pos = {int(s): j for j, s in enumerate(idx[0, 0]) if s >= 0}
    for s, src in pairs:
        if s in pos and src in pos:
            assert pos[src] < pos[s]


def test_fp32_evaluation_stays_inside_error_bound():
    """A sequential float32 evaluation of the score (the same formula, ordinary
    rounding) stays within the forward-error bound the oracle reports."""
    spec, x = _small_inputs(seed=9)
    qb, kb, w = bits(x["q"]), bits(x["kc"]), x["w"].numpy()
    rows = list(range(30, 96))
    exact = oracle.score_rows(qb, kb, w, 4, rows=rows)
    bound = oracle.score_error_bound(qb, kb, w, 4, rows=rows)
    qf = x["q"][0].float().numpy()
    kf = x["kc"][0].float().numpy()
    for i, t in enumerate(rows):
        n = oracle.visible_count(t, 4, spec.T)
        for s in range(n):
            acc = np.float32(0)
            for h in range(spec.H):
                z = np.float32(0)
                for d in range(spec.D):
                    z = np.float32(z + np.float32(qf[t, h, d] * kf[s, d]))
                acc = np.float32(acc + np.float32(w[0, t, h] * max(z, np.float32(0))))
            assert abs(float(acc) - exact[i, s]) <= bound[i, s]


def _worst_case_inputs(H, D=128, kc_dtype="bf16"):
    """A score whose sequential fp32 evaluation loses half an ulp at every addition.

    Head 0: q = (1, 2^-12, ..., 2^-12), key = (1, 2^-12, ..., 2^-12), w = 1, so its dot is
    1 + (D-1) 2^-24 and each of the D-1 small products (2^-24, half an ulp of 1) rounds
    away (round to nearest even).  Heads 1..H-1: q = 2^-12 e_0 and w = 2^-12, so each
    adds 2^-24 to a running sum of 1 and rounds away again.  The exact score is
    1 + (D + H - 2) 2^-24, the fp32 one is 1: the error is (D + H - 2) 2^-24.  With E4M3
    keys the small key entries are the smallest subnormal 2^-9 (byte 0x01), q's small
    entries 2^-15, and the key scale 1.0, so every product is the same."""
    q = np.zeros((1, 1, H, D), dtype=np.float32)
    w = np.zeros((1, 1, H), dtype=np.float32)
    small_q = 2.0 ** -12 if kc_dtype == "bf16" else 2.0 ** -15
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 0, 1:] = small_q
    w[0, 0, 0] = 1.0
    for h in range(1, H):
        q[0, 0, h, 0] = 2.0 ** -12
        w[0, 0, h] = 2.0 ** -12
    qb = bits(torch.from_numpy(q).to(torch.bfloat16))
    if kc_dtype == "bf16":
        k = np.full((1, 1, D), 2.0 ** -12, dtype=np.float32)
        k[0, 0, 0] = 1.0
        kb, ks = bits(torch.from_numpy(k).to(torch.bfloat16)), None
    else:
        kb = np.full((1, 1, D), 0x01, dtype=np.uint8)       # 2^-9
        kb[0, 0, 0] = 0x38                                   # 1.0 (exponent 7 = bias)
        ks = np.ones((1, 1), dtype=np.float32)
    return qb, kb, w, ks


def _sequential_fp32(qb, kb, w, kc_dtype="bf16", ks=None):
    """The score of query 0 and key 0 evaluated in fp32 the plain way: each dot product
    summed left to right with fp32 rounding, then acc = fma(w_h, max(z_h, 0), acc)."""
    qf = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).float().numpy()[0, 0]
    if kc_dtype == "bf16":
        kf = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).float().numpy()[0, 0]
    else:
        kf = torch.from_numpy(kb).view(torch.float8_e4m3fn).float().numpy()[0, 0]
    H, D = qf.shape
    acc = np.float32(0)
    for h in range(H):
        z = np.float32(0)
        for d in range(D):
            z = np.float32(z + np.float32(qf[h, d] * kf[d]))
        if ks is not None:
            z = np.float32(z * np.float32(ks[0, 0]))
        # fma: the float64 product and sum of these values are exact; one rounding
        acc = np.float32(np.float64(w[0, 0, h]) * np.float64(max(z, np.float32(0)))
                         + np.float64(acc))
    return float(acc)


@pytest.mark.parametrize("kc_dtype", ["bf16", "e4m3fn"])
@pytest.mark.parametrize("H", [1, 8, 64])
def test_error_bound_is_tight_on_worst_case(H, kc_dtype):
    """The fp32 forward-error bound is reached to within a few percent by a
    constructed worst case, so it is neither loose nor too tight: a bound scaled by
    2 or by 1/2 fails here."""
    D = 128
    qb, kb, w, ks = _worst_case_inputs(H, D, kc_dtype)
    exact = oracle.score_rows(qb, kb, w, 1, kc_dtype=kc_dtype, kc_scale=ks)[0, 0]
    beta = oracle.score_error_bound(qb, kb, w, 1, kc_dtype=kc_dtype, kc_scale=ks)[0, 0]
    got = _sequential_fp32(qb, kb, w, kc_dtype, ks)
    u = 2.0 ** -24
    assert exact == 1.0 + (D + H - 2) * u                   # exact in float64
    assert got == 1.0
    err = exact - got
    assert err <= beta
    assert err >= 0.95 * beta, (err / beta)


def test_error_bound_closed_form_all_ones():
    """All-ones q, keys and weights: sum_h |w_h| sum_d |q k| = H D, so the bound is
    (D + H + 2) 2^-24 H D."""
    for H in (1, 3, 64):
        D = 128
        qb = bits(torch.ones((1, 1, H, D), dtype=torch.bfloat16))
        kb = bits(torch.ones((1, 2, D), dtype=torch.bfloat16))
        w = np.ones((1, 1, H), dtype=np.float32)
        beta = oracle.score_error_bound(qb, kb, w, 1, q_pos0=1)[0]
        assert (beta == (D + H + 2) * 2.0 ** -24 * H * D).all()


@pytest.mark.parametrize("m,q_pos0,S,T", [(1, 0, 9, 9), (4, 0, 40, 10), (4, 5, 23, 12),
                                          (3, 0, 20, 4), (2, 7, 15, 30)])
def test_score_rows_mask_matches_brute_force(m, q_pos0, S, T):
    """-inf exactly where (s + 1) m > t + 1 for the absolute position t = q_pos0 + row
    (brute force over every (row, key) pair), finite everywhere else."""
    spec = synth.InputSpec(B=1, S=S, T=T, H=2, D=128, m=m, k=4, seed=31)
    x = synth.make_inputs(spec)
    rows = oracle.score_rows(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), m, q_pos0=q_pos0)
    want = np.zeros((S, T), dtype=bool)
    for r in range(S):
        for s in range(T):
            want[r, s] = (s + 1) * m > q_pos0 + r + 1
    assert (np.isneginf(rows) == want).all()
    assert np.isfinite(rows[~want]).all()


# ---------------------------------------------------------------------------
# Planted mistakes: every one must be caught by a pin above
# ---------------------------------------------------------------------------

def _no_relu(q_row, w_row, keys, scale):
    return w_row @ ((q_row @ keys.T) * scale[None, :])


def _relu_after_weight(q_row, w_row, keys, scale):
    return np.maximum(w_row[:, None] * ((q_row @ keys.T) * scale[None, :]), 0.0).sum(0)


def _no_scale(q_row, w_row, keys, scale):
    return w_row @ np.maximum(q_row @ keys.T, 0.0)


def _mask_off_by_one(t_abs, m, T):
    return max(0, min(T, (t_abs + 2) // m))


def _higher_index_first(scores, k):
    n = scores.shape[0]
    order = np.lexsort((-np.arange(n), -scores))
    keep = order[: min(k, n)]
    idx = np.full(k, -1, dtype=np.int64)
    val = np.full(k, -np.inf)
    idx[: keep.shape[0]] = keep
    val[: keep.shape[0]] = scores[keep]
    return idx, val


def _bad_bias_table():
    t = OI.E4M3FN_TABLE.copy()
    return t * 2.0


def _bound_scaled(factor):
    orig = OI.score_error_bound

    def f(*a, **kw):
        return orig(*a, **kw) * factor
    return f


def _run_pins(pins):
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    return caught


def _hand_pins():
    return [lambda c=c: _check_hand(c) for c in CASES]


def _bound_pins():
    return [lambda H=H, dt=dt: test_error_bound_is_tight_on_worst_case(H, dt)
            for H in (1, 8, 64) for dt in ("bf16", "e4m3fn")]


def _mask_pins():
    return [lambda: test_score_rows_mask_matches_brute_force(4, 5, 23, 12),
            lambda: test_score_rows_mask_matches_brute_force(3, 0, 20, 4)]


@pytest.mark.parametrize("mutant", ["no_relu", "relu_after_weight", "no_scale",
                                    "mask_off_by_one", "higher_index_first", "e4m3_bias",
                                    "bound_x2", "bound_half", "bound_no_head_term"])
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    pins = _hand_pins()
    if mutant == "no_relu":
        monkeypatch.setattr(OI, "score_row", _no_relu)
    elif mutant == "relu_after_weight":
        monkeypatch.setattr(OI, "score_row", _relu_after_weight)
    elif mutant == "no_scale":
        monkeypatch.setattr(OI, "score_row", _no_scale)
    elif mutant == "mask_off_by_one":
        monkeypatch.setattr(OI, "visible_count", _mask_off_by_one)
        # the mask of the written score rows is pinned on its own as well
        assert _run_pins(_mask_pins()) > 0
    elif mutant == "higher_index_first":
        monkeypatch.setattr(OI, "select_topk", _higher_index_first)
    elif mutant == "e4m3_bias":
        monkeypatch.setattr(OI, "E4M3FN_TABLE", _bad_bias_table())
    elif mutant == "bound_x2":
        monkeypatch.setattr(OI, "score_error_bound", _bound_scaled(2.0))
        monkeypatch.setattr(oracle, "score_error_bound", OI.score_error_bound)
        pins = _bound_pins()
    elif mutant == "bound_half":
        monkeypatch.setattr(OI, "score_error_bound", _bound_scaled(0.5))
        monkeypatch.setattr(oracle, "score_error_bound", OI.score_error_bound)
        pins = _bound_pins()
    elif mutant == "bound_no_head_term":
        # a bound that forgets the head sum's additions: (D + 2) instead of (D + H + 2)
        orig = OI.score_error_bound

        def no_head(q_bits, kc_bits, w, m, **kw):
            H = np.asarray(q_bits).shape[2]
            return orig(q_bits, kc_bits, w, m, **kw) * (128 + 2) / (128 + H + 2)
        monkeypatch.setattr(oracle, "score_error_bound", no_head)
        pins = _bound_pins()
    assert _run_pins(pins) > 0, mutant
