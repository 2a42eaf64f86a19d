"""GPU parity of the two-stage (coarse -> fine) indexer.

* Block keys: bit for bit against the oracle's.
* Every block kept (a query sees at most k_blocks complete blocks): bit for bit equal
  to the single-stage indexer.
* Lossy coarse stage: the coarse stage is the single-stage indexer on block keys, so
  its kept blocks are checked against the float64 oracle of that problem; the fine
  stage is checked against the float64 oracle over the GPU's own candidate set (the
  kept blocks' keys plus the trailing keys); scores within the fp32 bound; end-to-end
  recall against the oracle's own two-stage result is reported.
* Bit for bit against a materialise-then-select of the same candidates: the fine
  scores equal the written score rows of si_materialize_scores, and the top-k of those
  rows restricted to the candidates is the output.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hand import bits
from parity import assert_same, check_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run(si, x, kb, m, k, **kw):
    out = si.indexer_topk_two_stage(x["q"], x["kc"], kb, x["w"], m, k, **kw)
    torch.cuda.synchronize()
    return out


def candidates(coarse_idx_row, t_abs, m, T, block, k_blocks):
    """The fine candidate keys of one row from its kept blocks (GPU coarse output)."""
    n = oracle.visible_count(t_abs, m, T)
    nb = oracle.visible_count(t_abs, block * m, T // block)
    blocks = np.asarray(coarse_idx_row[:min(nb, k_blocks)], dtype=np.int64)
    assert (blocks >= 0).all() and (blocks < nb).all()
    c = (block * blocks[:, None] + np.arange(block)[None, :]).reshape(-1)
    return np.concatenate([c, np.arange(block * nb, n)])


def check_fine(gi, gs, rows, cand_lists, exact, beta, k):
    """Fine stage vs the float64 oracle restricted to each row's candidates: the
    the benchmark spec rules (recall, mismatches at the k-th score, scores within beta)."""
    recalls = []
    for i, _ in enumerate(rows):
        c = cand_lists[i]
        need = min(k, c.size)
        g = np.asarray(gi[i][:need], dtype=np.int64)
        assert (np.asarray(gi[i][need:]) == -1).all() and np.isneginf(gs[i][need:]).all()
        assert set(g.tolist()) <= set(c.tolist()), "selected key outside the candidates"
        if need == 0:
            continue
        sc = exact[i, c]
        order = np.lexsort((c, -sc))[:need]
        O, G = set(c[order].tolist()), set(g.tolist())
        recalls.append(len(O & G) / need)
        skth = sc[order[-1]]
        for s in O ^ G:
            gap = abs(exact[i, s] - skth)
            assert gap <= 1e-3 * abs(skth) or gap <= 2 * beta[i, s], (i, s, gap)
        err = np.abs(np.asarray(gs[i][:need], dtype=np.float64) - exact[i, g])
        assert (err <= beta[i, g]).all(), "fine score outside the fp32 bound"
    mean = float(np.mean(recalls)) if recalls else 1.0
    assert mean >= 0.998, mean
    return mean


@pytest.mark.parametrize("block", [4, 8, 16])
def test_block_keys_bit_exact(gpu_lib, block):
    rnd = np.random.default_rng(block)
    kc = torch.from_numpy((rnd.standard_normal((2, 1003, 128)) *
                           10.0 ** rnd.uniform(-3, 3, (2, 1003, 1))).astype(np.float32)).to(torch.bfloat16)
    kb = gpu_lib.block_keys(kc.to(DEV), block)
    torch.cuda.synchronize()
    want = oracle.block_keys_mean(bits(kc), block)
    assert kb.shape == (2, 1003 // block, 128)
    assert (kb.cpu().view(torch.int16).numpy().view(np.uint16) == want).all()


@pytest.mark.parametrize("q_pos0", [0, 37])
def test_every_block_kept_equals_single_stage(gpu_lib, q_pos0):
    spec = synth.InputSpec(B=2, S=2000, T=500, H=64, m=4, k=64, seed=31)
    say("two-stage all blocks kept", q_pos0)
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], 8)
    ts = run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=2048, q_pos0=q_pos0)
    ref = gpu_lib.indexer_topk(x["q"], x["kc"], x["w"], spec.m, spec.k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert_same(ts, ref, "two-stage with every block kept vs single-stage")


def _lossy_case(gpu_lib, spec, block, k_blocks, q_pos0=0, **kw):
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], block)
    gi, gs = run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=k_blocks, block=block, q_pos0=q_pos0,
                 **kw)
    # the coarse stage is the single-stage indexer on the block keys (same kernels)
    ci, cs = gpu_lib.indexer_topk(x["q"], kb, x["w"], block * spec.m, k_blocks, q_pos0=q_pos0)
    torch.cuda.synchronize()
    return x, kb, (gi, gs), (ci, cs)


def test_lossy_two_stage_vs_oracle(gpu_lib):
    spec = synth.InputSpec(B=1, S=3000, T=3000, H=64, m=1, k=128, seed=32)
    block, k_blocks = 8, 48
    say("two-stage lossy", spec, block, k_blocks)
    x, kb, (gi, gs), (ci, cs) = _lossy_case(gpu_lib, spec, block, k_blocks)
    qb, kcb, w = bits(x["q"]), bits(x["kc"]), x["w"].cpu().numpy()
    rows = list(range(0, spec.S, 7)) + [spec.S - 1]
    # coarse stage against the float64 oracle of the block-key problem
    kbb = bits(kb)
    st = check_rows(ci[0].cpu().numpy()[rows], cs[0].cpu().numpy()[rows], rows, qb, kbb, w,
                    block * spec.m, k_blocks)
    say("coarse vs oracle", st)
    assert (kbb == oracle.block_keys_mean(kcb, block)).all()
    # fine stage against the float64 oracle over the GPU's candidates
    exact = oracle.score_rows(qb, kcb, w, spec.m, rows=rows)
    beta = oracle.score_error_bound(qb, kcb, w, spec.m, rows=rows)
    cin = ci[0].cpu().numpy()
    cands = [candidates(cin[r], r, spec.m, spec.T, block, k_blocks) for r in rows]
    gin, gsn = gi[0].cpu().numpy()[rows], gs[0].cpu().numpy()[rows]
    mean = check_fine(gin, gsn, rows, cands, exact, beta, spec.k)
    # end to end against the oracle's own two-stage selection (reported)
    oi, _ = oracle.two_stage_topk(qb, kcb, w, spec.m, spec.k, k_blocks=k_blocks, block=block,
                                  rows=rows)
    rec = []
    for i, r in enumerate(rows):
        need = min(spec.k, int((oi[0, i] >= 0).sum()))
        if need:
            rec.append(len(set(gin[i][:need]) & set(oi[0, i][:need])) / need)
    say(f"fine recall {mean:.4f}; end-to-end recall vs the oracle's two-stage "
        f"{np.mean(rec):.4f} (min {np.min(rec):.4f})")
    assert np.mean(rec) >= 0.998


def test_two_stage_bit_exact_vs_materialize(gpu_lib):
    """The fine scores are the single-stage scores bit for bit, and the output is the
    top-k of the written score rows restricted to the candidates."""
    spec = synth.InputSpec(B=2, S=1500, T=1500, H=64, m=1, k=100, seed=33)
    block, k_blocks = 8, 40
    say("two-stage vs materialise", spec)
    x, kb, (gi, gs), (ci, cs) = _lossy_case(gpu_lib, spec, block, k_blocks, q_pos0=11)
    sc = gpu_lib.materialize_scores(x["q"], x["kc"], x["w"], spec.m, q_pos0=11)
    torch.cuda.synchronize()
    scn = sc.cpu().numpy()
    for b in range(spec.B):
        gin, gsn, cin = gi[b].cpu().numpy(), gs[b].cpu().numpy(), ci[b].cpu().numpy()
        for r in range(spec.S):
            c = candidates(cin[r], 11 + r, spec.m, spec.T, block, k_blocks)
            need = min(spec.k, c.size)
            v = scn[b, r, c]
            # selection by (score desc, index asc) on the GPU's own fp32 scores
            order = np.lexsort((c, -v.astype(np.float64)))[:need]
            assert (gin[r, :need] == c[order]).all(), (b, r)
            assert (gsn[r, :need].view(np.uint32) == v[order].view(np.uint32)).all(), (b, r)
            assert (gin[r, need:] == -1).all()


def test_two_stage_knobs_bit_identical(gpu_lib):
    spec = synth.InputSpec(B=1, S=2500, T=2500, H=64, m=1, k=64, seed=34)
    say("two-stage knobs")
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], 8)
    base = run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=32)
    for kw in (dict(query_chunk=96), dict(query_chunk=1000), dict(key_tile=64),
               dict(key_tile=256, key_partition=256), dict(query_chunk=2500, key_tile=1024)):
        assert_same(run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=32, **kw), base, str(kw))


def test_two_stage_several_coarse_chunks(gpu_lib):
    """S = 33,000: the coarse indexer runs over coarse chunks of up to 32,768 rows (two
    here, the second ragged), the fine stage over query chunks inside them.  The output
    does not depend on how the rows are chunked, and rows on both sides of the coarse
    boundary match the oracle's two-stage result."""
    spec = synth.InputSpec(B=1, S=33000, T=2000, H=8, m=16, k=64, seed=36)
    say("two-stage several coarse chunks", spec)
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], 8)
    base = run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=32)
    for kw in (dict(query_chunk=96), dict(query_chunk=33000), dict(query_chunk=5000)):
        assert_same(run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=32, **kw), base, str(kw))
    rows = [0, 1, 4095, 4096, 32735, 32736, 32767, 32768, 32769, 32999]
    oi, ov = oracle.two_stage_topk(bits(x["q"]), bits(x["kc"]), x["w"].cpu().numpy(), spec.m,
                                   spec.k, k_blocks=32, block=8, rows=rows)
    gin = base[0][0].cpu().numpy()
    for i, r in enumerate(rows):
        n = int((oi[0, i] >= 0).sum())
        assert int((gin[r] >= 0).sum()) == n, r
        assert len(set(gin[r, :n]) & set(oi[0, i, :n])) >= n - 1, r


@pytest.mark.parametrize("pattern", ["constant", "two-valued"])
def test_two_stage_fine_select_fallbacks(gpu_lib, pattern):
    """Fine selection's radix path: every key equal (a row's candidate scores have no
    range) or keys alternating between two values (the k-th key's score bin holds far
    more than 64 candidates).  Ties then decide most of the selection, by index in both
    stages; the result equals the oracle's two-stage top-k index for index."""
    spec = synth.InputSpec(B=1, S=1200, T=1200, H=8, m=1, k=100, seed=37)
    say("two-stage fine-select fallback", pattern)
    x = synth.make_inputs(spec)
    kc = x["kc"].clone()
    if pattern == "constant":
        kc[0, :] = kc[0, 0]
    else:
        kc[0, 0::2] = kc[0, 0]
        kc[0, 1::2] = kc[0, 1]
    x = dict(x, kc=kc)
    xd = {key: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for key, v in x.items()}
    kb = gpu_lib.block_keys(xd["kc"], 8)
    gi, gs = run(gpu_lib, xd, kb, spec.m, spec.k, k_blocks=32)
    rows = [0, 99, 100, 263, 264, 700, spec.S - 1]
    oi, _ = oracle.two_stage_topk(bits(x["q"]), bits(kc), x["w"].numpy(), spec.m, spec.k,
                                  k_blocks=32, block=8, rows=rows)
    gin = gi[0].cpu().numpy()
    for i, r in enumerate(rows):
        np.testing.assert_array_equal(gin[r], oi[0, i], err_msg=f"{pattern} row {r}")


@pytest.mark.parametrize("T,k,k_blocks,block", [(5, 8, 4, 8), (300, 2048, 2048, 8),
                                                (900, 1, 1, 8), (700, 700, 3, 32)])
def test_two_stage_edge_cases(gpu_lib, T, k, k_blocks, block):
    """No complete block (T < block), k larger than every candidate set, a single kept
    block and k = 1, large blocks: against the oracle row by row."""
    spec = synth.InputSpec(B=1, S=min(4 * T + 40, 2000), T=T, H=8, m=4, k=k, seed=35)
    say("two-stage edge", T, k, k_blocks, block)
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], block)
    gi, gs = run(gpu_lib, x, kb, spec.m, k, k_blocks=k_blocks, block=block)
    oi, ov = oracle.two_stage_topk(bits(x["q"]), bits(x["kc"]), x["w"].cpu().numpy(), spec.m, k,
                                   k_blocks=k_blocks, block=block)
    gin = gi[0].cpu().numpy()
    for r in range(spec.S):
        n = int((oi[0, r] >= 0).sum())
        assert int((gin[r] >= 0).sum()) == n, r
        if n:
            assert len(set(gin[r, :n]) & set(oi[0, r, :n])) >= n - 1, r


@pytest.mark.slow
def test_two_stage_long_context(gpu_lib):
    """S = 262,144, T = 65,536: 8,192 blocks of 8, the page's 2,048 kept, top-512."""
    spec = synth.CONFIGS["long"]
    say("two-stage long", spec)
    x = synth.make_inputs(spec, device=DEV)
    kb = gpu_lib.block_keys(x["kc"], 8)
    gi, gs = run(gpu_lib, x, kb, spec.m, spec.k, k_blocks=2048)
    # rows that see more than 2,048 complete blocks (the coarse stage drops blocks)
    rows = synth.sample_rows(spec.replace(k=8 * 2048), 64)
    idx = torch.as_tensor(rows, device=DEV)
    qb = bits(x["q"][:, idx])
    kcb = bits(x["kc"])
    w = x["w"][:, idx].cpu().numpy()
    # fine stage against the oracle over the GPU's candidates; each row's coarse blocks
    # come from the indexer on the block keys at the row's own offset (the same kernels
    # the two-stage driver runs)
    recs = []
    for i, r in enumerate(rows):
        cir, _ = gpu_lib.indexer_topk(x["q"][:, r:r + 1].contiguous(), kb,
                                      x["w"][:, r:r + 1].contiguous(), 8 * spec.m, 2048, q_pos0=r)
        torch.cuda.synchronize()
        c = candidates(cir[0, 0].cpu().numpy(), r, spec.m, spec.T, 8, 2048)
        n = oracle.visible_count(r, spec.m, spec.T)
        ex = oracle.score_rows(qb[:, i:i + 1], kcb[:, :n], w[:, i:i + 1], spec.m, q_pos0=r)
        bt = oracle.score_error_bound(qb[:, i:i + 1], kcb[:, :n], w[:, i:i + 1], spec.m, q_pos0=r)
        recs.append(check_fine(gi[0, r:r + 1].cpu().numpy(), gs[0, r:r + 1].cpu().numpy(), [r],
                               [c], ex, bt, spec.k))
    say(f"two-stage long: {len(rows)} rows, fine recall mean {np.mean(recs):.4f}")
