"""GPU parity of the sparse-attention consumer: element by element against the
float64 oracle within the error bound derived from the GPU arithmetic, on the same
selected indices; the composition indexer -> attention against the oracle pipeline."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hand import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check_attention(out, qa, kv, idx, scale, rows=None):
    """out [B, S, HA, D] (GPU, bf16) against the oracle on the same idx."""
    qb, kb, ix = bits(qa), bits(kv), idx.cpu().numpy()
    o = oracle.sparse_attention(qb, kb, ix, scale, rows=rows)
    beta = oracle.attention_error_bound(qb, kb, ix, scale, rows=rows)
    g = out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[:, rows]
    err = np.abs(g - o)
    assert (err <= beta).all(), f"max excess {(err - beta).max()} worst ratio {(err / np.maximum(beta, 1e-300)).max()}"
    return float((err / np.maximum(beta, 1e-300)).max())


def random_selection(rnd, B, S, T, k, counts):
    """idx [B, S, k]: row t selects counts[t % len(counts)] distinct keys, -1 after."""
    idx = np.full((B, S, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(S):
            n = min(counts[t % len(counts)], k, T)
            idx[b, t, :n] = rnd.permutation(T)[:n]
    return torch.from_numpy(idx)


@pytest.mark.parametrize("HA,k", [(64, 64), (32, 512), (96, 100), (128, 33)])
def test_attention_vs_oracle(gpu_lib, HA, k):
    rnd = np.random.default_rng(HA + k)
    spec = synth.InputSpec(B=2, S=96, T=700, H=4, m=4, k=k, seed=41)
    qa, kv = synth.gen_attention_inputs(spec, HA)
    idx = random_selection(rnd, 2, 96, 700, k, [k, 0, 1, 31, 32, 33, 65, k - 1])
    scale = oracle.default_scale(128)
    out = gpu_lib.sparse_attention(qa.to(DEV), kv.to(DEV), idx.to(DEV), scale)
    torch.cuda.synchronize()
    worst = check_attention(out, qa, kv, idx, scale)
    say(f"attention HA={HA} k={k}: worst error / bound {worst:.3f}")
    # rows with nothing selected are zeros
    assert (out[:, 1::8].float() == 0).all()


def test_attention_large_logits_and_scale(gpu_lib):
    """Logits far from zero (scale 1, large q): the running maximum keeps exp2 in range."""
    rnd = np.random.default_rng(3)
    spec = synth.InputSpec(B=1, S=40, T=300, H=4, m=4, k=128, seed=42)
    qa, kv = synth.gen_attention_inputs(spec, 64)
    qa = (qa.float() * 8).to(torch.bfloat16)
    idx = random_selection(rnd, 1, 40, 300, 128, [128, 77])
    out = gpu_lib.sparse_attention(qa.to(DEV), kv.to(DEV), idx.to(DEV), 1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    check_attention(out, qa, kv, idx, 1.0)


def test_attention_list_ends_at_first_invalid_index(gpu_lib):
    rnd = np.random.default_rng(4)
    spec = synth.InputSpec(B=1, S=4, T=200, H=4, m=4, k=96, seed=43)
    qa, kv = synth.gen_attention_inputs(spec, 64)
    idx = random_selection(rnd, 1, 4, 200, 96, [96])
    bad = idx.clone()
    bad[0, 0, 40] = -1          # the list of row 0 ends at 40
    bad[0, 1, 70] = 200         # out of range ends row 1 at 70
    bad[0, 2, 0] = -7           # row 2 selects nothing
    cut = idx.clone()
    cut[0, 0, 40:] = -1
    cut[0, 1, 70:] = -1
    cut[0, 2, :] = -1
    a = gpu_lib.sparse_attention(qa.to(DEV), kv.to(DEV), bad.to(DEV))
    b = gpu_lib.sparse_attention(qa.to(DEV), kv.to(DEV), cut.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_composition_indexer_then_attention(gpu_lib):
    """indexer_topk -> sparse_attention on the tiny indexer: the attention output matches
    the oracle on the GPU's own selection, and the oracle pipeline's selection (float64
    indexer) gives the same rows wherever the two selections agree."""
    spec = synth.CONFIGS["tiny"]
    say("composition tiny")
    x = synth.make_inputs(spec)
    qa, kv = synth.gen_attention_inputs(spec, 64)
    xd = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    gi, _ = gpu_lib.indexer_topk(xd["q"], xd["kc"], xd["w"], spec.m, spec.k)
    out = gpu_lib.sparse_attention(qa.to(DEV), kv.to(DEV), gi)
    torch.cuda.synchronize()
    scale = oracle.default_scale(spec.D)
    check_attention(out, qa, kv, gi, scale)
    oi, _ = oracle.indexer_topk(bits(x["q"]), bits(x["kc"]), x["w"].numpy(), spec.m, spec.k)
    gin = gi.cpu().numpy()
    same = [t for t in range(spec.S) if set(gin[0, t]) == set(oi[0, t])]
    say(f"composition: {len(same)} of {spec.S} rows select the oracle's exact set")
    assert len(same) >= 0.99 * spec.S


@pytest.mark.slow
def test_composition_long_context(gpu_lib):
    """S = 262,144: the streaming indexer feeding the attention (the pages' composition
    shape), sampled rows against the oracle attention on the GPU's selection."""
    spec = synth.CONFIGS["long"]
    say("composition long")
    x = synth.make_inputs(spec, device=DEV)
    qa, kv = synth.gen_attention_inputs(spec, 64, device=DEV)
    torch.cuda.synchronize()
    gi, _ = gpu_lib.indexer_topk(x["q"], x["kc"], x["w"], spec.m, spec.k)
    out = gpu_lib.sparse_attention(qa, kv, gi)
    torch.cuda.synchronize()
    rows = synth.sample_rows(spec, 48)
    ridx = torch.as_tensor(rows, device=DEV)
    worst = check_attention(out[:, ridx], qa[:, ridx], kv, gi[:, ridx], oracle.default_scale(128))
    say(f"composition long: {len(rows)} rows, worst error / bound {worst:.3f}")
