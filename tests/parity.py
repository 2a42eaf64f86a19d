"""Comparison of GPU top-k rows with the float64 oracle, with the stated tolerances.

For each checked query row t (G = GPU index set, O = oracle index set, padding
excluded, s*_k = the oracle's k-th score):
  * |G| == |O| == min(k, n_t), and the padding is exactly -1 / -inf;
  * recall r_t = |G & O| / |O|; the gate is mean recall >= 0.998 over the checked rows;
  * every key in G ^ O has an oracle score within 1e-3 * |s*_k| of s*_k, or within
    2 * beta (beta = fp32 forward-error bound of that score);
  * every GPU score is within max(1e-3 * |oracle|, beta) of the oracle's score of the
    same key, and within beta outright (the stronger check, also reported);
  * the GPU row is sorted by (score desc, idx asc) of its own scores.
"""

from __future__ import annotations

import math

import numpy as np

import oracle


def check_rows(gidx, gscore, rows, q_bits, kc_bits, w, m, k, *, kc_dtype="bf16",
               kc_scale=None, q_pos0=0, b=0, recall_gate=0.998, verbose=True, q_dtype="bf16"):
    """gidx/gscore: [R, k] numpy GPU outputs for the query rows `rows` of batch b."""
    rows = list(rows)
    exact = oracle.score_rows(q_bits, kc_bits, w, m, kc_dtype=kc_dtype, kc_scale=kc_scale,
                              q_pos0=q_pos0, rows=rows, b=b, q_dtype=q_dtype)
    beta = oracle.score_error_bound(q_bits, kc_bits, w, m, kc_dtype=kc_dtype,
                                    kc_scale=kc_scale, q_pos0=q_pos0, rows=rows, b=b,
                                    q_dtype=q_dtype)
    T = exact.shape[1]
    recalls = []
    worst_rel = 0.0
    floor_used = 0
    mismatches = 0
    for i, t in enumerate(rows):
        n = oracle.visible_count(q_pos0 + t, m, T)
        need = min(k, n)
        gi = np.asarray(gidx[i], dtype=np.int64)
        gs = np.asarray(gscore[i], dtype=np.float64)
        assert (gi[need:] == -1).all() and np.isneginf(gs[need:]).all(), f"row {t}: padding"
        assert (gi[:need] >= 0).all() and (gi[:need] < n).all(), f"row {t}: index out of range"
        assert len(set(gi[:need].tolist())) == need, f"row {t}: duplicate index"
        # own order: score desc, index asc
        for j in range(need - 1):
            assert (gs[j] > gs[j + 1]) or (gs[j] == gs[j + 1] and gi[j] < gi[j + 1]), \
                f"row {t}: not sorted at {j}"
        if need == 0:
            continue
        oi, _ = oracle.select_topk(exact[i, :n], k)
        O = set(oi[:need].tolist())
        G = set(gi[:need].tolist())
        recalls.append(len(G & O) / len(O))
        mismatches += len(G ^ O) // 2
        skth = exact[i, oi[need - 1]]
        for s in G ^ O:
            gap = abs(exact[i, s] - skth)
            if gap > 1e-3 * abs(skth):
                # the floor only decides where the relative rule is narrower than it
                assert 1e-3 * abs(skth) < 2 * beta[i, s], f"row {t}: floor used needlessly"
                assert gap <= 2 * beta[i, s], f"row {t}: mismatch key {s} gap {gap}"
                floor_used += 1
        ex = exact[i, gi[:need]]
        err = np.abs(gs[:need] - ex)
        bnd = beta[i, gi[:need]]
        assert (err <= np.maximum(1e-3 * np.abs(ex), bnd)).all(), f"row {t}: score tolerance"
        assert (err <= bnd).all(), f"row {t}: score outside fp32 error bound"
        rel = err / np.maximum(np.abs(ex), 1e-30)
        worst_rel = max(worst_rel, float(rel.max()))
    mean_recall = float(np.mean(recalls)) if recalls else 1.0
    assert mean_recall >= recall_gate, f"mean recall {mean_recall}"
    stats = {"mean_recall": mean_recall, "min_recall": float(min(recalls)) if recalls else 1.0,
             "rows": len(rows), "floor_used": floor_used, "worst_rel_err": worst_rel,
             "mismatches": mismatches}
    if verbose:
        print("[parity]", stats, flush=True)
    return stats


def check_score_block(gscores, rows, q_bits, kc_bits, w, m, *, kc_dtype="bf16", kc_scale=None,
                      q_pos0=0, b=0, q_dtype="bf16"):
    """Element-by-element check of written scores [R, T]: -inf exactly where masked,
    within the fp32 error bound of the float64 score elsewhere."""
    rows = list(rows)
    exact = oracle.score_rows(q_bits, kc_bits, w, m, kc_dtype=kc_dtype, kc_scale=kc_scale,
                              q_pos0=q_pos0, rows=rows, b=b, q_dtype=q_dtype)
    beta = oracle.score_error_bound(q_bits, kc_bits, w, m, kc_dtype=kc_dtype,
                                    kc_scale=kc_scale, q_pos0=q_pos0, rows=rows, b=b,
                                    q_dtype=q_dtype)
    g = np.asarray(gscores, dtype=np.float64)
    masked = np.isneginf(exact)
    assert (np.isneginf(g) == masked).all(), "mask differs"
    vis = ~masked
    err = np.abs(g[vis] - exact[vis])
    assert (err <= beta[vis]).all(), f"score outside bound: max excess {(err - beta[vis]).max()}"
    # no negative zero ever reaches the output
    assert not (np.signbit(g[vis]) & (g[vis] == 0)).any()
    return float(err.max()) if err.size else 0.0


def assert_same(a, b, what=""):
    """Bit-exact equality of two (idx, score) GPU results."""
    ai, as_ = (x.cpu() for x in a)
    bi, bs = (x.cpu() for x in b)
    assert ai.shape == bi.shape
    assert (ai == bi).all().item(), f"{what}: indices differ"
    av = as_.view(dtype=ai.dtype)  # compare score bits
    bv = bs.view(dtype=bi.dtype)
    assert (av == bv).all().item(), f"{what}: score bits differ"


def pairs(S, T, m, q_pos0=0):
    return sum(min(T, (q_pos0 + t + 1) // m) for t in range(S))


NEG_INF = -math.inf
