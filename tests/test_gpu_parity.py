"""GPU parity: the HIP path against the float64 oracle and against its own
materialise-then-select reference path, through the C ABI."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from hand import bits, build, expected, load_cases
from parity import assert_same, check_rows, check_score_block

pytestmark = pytest.mark.gpu
DEV = "cuda"
CASES = load_cases()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_stream(si, x, m, k, **kw):
    out = si.indexer_topk(x["q"], x["kc"], x["w"], m, k, kc_scale=x.get("kc_scale"), **kw)
    torch.cuda.synchronize()
    return out


def run_mat(si, x, m, k, **kw):
    out = si.materialize_topk(x["q"], x["kc"], x["w"], m, k, kc_scale=x.get("kc_scale"), **kw)
    torch.cuda.synchronize()
    return out


def oracle_args(xc, spec_or_case):
    kc_dtype = "e4m3fn" if xc["kc"].dtype == torch.uint8 else "bf16"
    return dict(q_bits=bits(xc["q"]), kc_bits=bits(xc["kc"]), w=xc["w"].cpu().numpy(),
                kc_dtype=kc_dtype,
                kc_scale=None if xc.get("kc_scale") is None else xc["kc_scale"].cpu().numpy())


# ---------------------------------------------------------------------------
# Hand cases: exact values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key_tile", [64, 512])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_cases_exact(gpu_lib, case, key_tile):
    say("hand", case["name"], key_tile)
    x = build(case)
    xd = dev(x)
    eidx, eval_ = expected(case)
    for out in (run_stream(gpu_lib, xd, x["m"], x["k"], q_pos0=x["q_pos0"], key_tile=key_tile),
                run_mat(gpu_lib, xd, x["m"], x["k"], q_pos0=x["q_pos0"])):
        np.testing.assert_array_equal(out[0].cpu().numpy(), eidx)
        np.testing.assert_array_equal(out[1].cpu().double().numpy(), eval_)
        # +0, never -0, for the all-zero row of H3
        assert not torch.signbit(out[1][out[1] == 0]).any()


# ---------------------------------------------------------------------------
# Tiny indexer (B=1, S=1024, T=256, k=64): every row against the oracle
# ---------------------------------------------------------------------------

def test_tiny_every_row(gpu_lib):
    spec = synth.CONFIGS["tiny"]
    say("tiny", spec)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    gi, gs = run_stream(gpu_lib, xd, spec.m, spec.k)
    st = check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S),
                    oa["q_bits"], oa["kc_bits"], oa["w"], spec.m, spec.k)
    say("tiny recall", st)
    mat = run_mat(gpu_lib, xd, spec.m, spec.k)
    assert_same((gi, gs), mat, "tiny stream vs materialise")
    sc = gpu_lib.materialize_scores(xd["q"], xd["kc"], xd["w"], spec.m)
    torch.cuda.synchronize()
    check_score_block(sc[0].cpu().numpy(), range(spec.S), oa["q_bits"], oa["kc_bits"], oa["w"],
                      spec.m)


# ---------------------------------------------------------------------------
# Ragged shapes: S, T not multiples of any tile, query offset, batch of 2
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("q_pos0", [0, 37])
def test_ragged_every_row(gpu_lib, q_pos0):
    spec = synth.InputSpec(B=2, S=1000, T=250, H=64, m=4, k=64, seed=21)
    say("ragged", q_pos0)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    gi, gs = run_stream(gpu_lib, xd, spec.m, spec.k, q_pos0=q_pos0)
    for b in range(spec.B):
        check_rows(gi[b].cpu().numpy(), gs[b].cpu().numpy(), range(spec.S), oa["q_bits"],
                   oa["kc_bits"], oa["w"], spec.m, spec.k, q_pos0=q_pos0, b=b)
    assert_same((gi, gs), run_mat(gpu_lib, xd, spec.m, spec.k, q_pos0=q_pos0), "ragged")
    sc = gpu_lib.materialize_scores(xd["q"], xd["kc"], xd["w"], spec.m, q_pos0=q_pos0,
                                    row0=333, rows=300)
    torch.cuda.synchronize()
    check_score_block(sc[1].cpu().numpy(), range(333, 633), oa["q_bits"], oa["kc_bits"],
                      oa["w"], spec.m, q_pos0=q_pos0, b=1)


@pytest.mark.parametrize("H,S,key_tile", [(3, 300, 512), (5, 1100, 512), (13, 700, 64),
                                          (128, 700, 512)])
def test_odd_heads_and_ratio(gpu_lib, H, S, key_tile):
    """Head counts that are not a multiple of 8 and the largest supported (128), m = 1
    (every earlier key visible), and rows whose keys span several register tiles."""
    spec = synth.InputSpec(B=1, S=S, T=S, H=H, m=1, k=100, seed=22 + H)
    say("odd heads", H, S, key_tile)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    gi, gs = run_stream(gpu_lib, xd, 1, 100, key_tile=key_tile)
    check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S), oa["q_bits"],
               oa["kc_bits"], oa["w"], 1, 100)
    assert_same((gi, gs), run_mat(gpu_lib, xd, 1, 100), "odd heads")


# ---------------------------------------------------------------------------
# E4M3 keys with a per-row scale
# ---------------------------------------------------------------------------

def test_e4m3_keys_every_row(gpu_lib):
    spec = synth.InputSpec(B=1, S=2048, T=512, H=64, m=4, k=64, seed=23, kc_dtype="e4m3fn")
    say("e4m3")
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    gi, gs = run_stream(gpu_lib, xd, spec.m, spec.k)
    check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S), oa["q_bits"],
               oa["kc_bits"], oa["w"], spec.m, spec.k, kc_dtype="e4m3fn",
               kc_scale=oa["kc_scale"])
    assert_same((gi, gs), run_mat(gpu_lib, xd, spec.m, spec.k), "e4m3")
    sc = gpu_lib.materialize_scores(xd["q"], xd["kc"], xd["w"], spec.m, kc_scale=xd["kc_scale"],
                                    row0=1500, rows=548)
    torch.cuda.synchronize()
    check_score_block(sc[0].cpu().numpy(), range(1500, 2048), oa["q_bits"], oa["kc_bits"],
                      oa["w"], spec.m, kc_dtype="e4m3fn", kc_scale=oa["kc_scale"])


def test_e4m3_every_code(gpu_lib):
    """Keys holding every finite E4M3 code at every byte position of a word (d mod 4),
    unit scales: the written scores against the oracle's own decoder, within beta,
    and the streamed top-k of every row."""
    spec = synth.InputSpec(B=1, S=256, T=256, H=4, m=1, k=32, seed=31, kc_dtype="e4m3fn")
    say("e4m3 every code")
    xc = synth.make_inputs(spec)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    s_idx = np.arange(spec.T)[:, None]
    d_idx = np.arange(128)[None, :]
    xc["kc"] = torch.from_numpy(codes[(s_idx + 7 * d_idx) % codes.size][None].copy())
    xc["kc_scale"] = torch.ones((1, spec.T), dtype=torch.float32)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    sc = gpu_lib.materialize_scores(xd["q"], xd["kc"], xd["w"], spec.m, kc_scale=xd["kc_scale"])
    torch.cuda.synchronize()
    check_score_block(sc[0].cpu().numpy(), range(spec.S), oa["q_bits"], oa["kc_bits"],
                      oa["w"], spec.m, kc_dtype="e4m3fn", kc_scale=oa["kc_scale"])
    gi, gs = run_stream(gpu_lib, xd, spec.m, spec.k)
    check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S), oa["q_bits"],
               oa["kc_bits"], oa["w"], spec.m, spec.k, kc_dtype="e4m3fn",
               kc_scale=oa["kc_scale"])


# ---------------------------------------------------------------------------
# Knob invariance: no tuning knob changes an output bit
# ---------------------------------------------------------------------------

def test_knobs_bit_identical(gpu_lib):
    spec = synth.InputSpec(B=2, S=2048, T=512, H=64, m=4, k=128, seed=24)
    say("knobs")
    xd = dev(synth.make_inputs(spec))
    ref = run_mat(gpu_lib, xd, spec.m, spec.k)
    for kt in (64, 128, 256, 512, 768, 1024):
        for qc in (0, 96, 512):
            for kp in (0, kt if kt >= 128 else 128):
                out = run_stream(gpu_lib, xd, spec.m, spec.k, key_tile=kt, query_chunk=qc,
                                 key_partition=kp)
                assert_same(out, ref, f"key_tile={kt} query_chunk={qc} key_partition={kp}")


@pytest.mark.parametrize("k", [1, 700, 1024, 2048])
def test_compaction_paths(gpu_lib, k):
    """Rows with 4096 visible keys: several in-kernel compactions for large k, the
    4096-slot buffer for k > 1024, partitions, and k above the visible count."""
    spec = synth.InputSpec(B=1, S=16384, T=4096, H=16, m=4, k=k, seed=25)
    say("compaction", k)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    ref = run_mat(gpu_lib, xd, spec.m, k)
    for kt, kp in ((512, 0), (1024, 0), (256, 2048 if k <= 2048 else 0)):
        if kp and (spec.T + kp - 1) // kp * k > 8192:
            continue
        out = run_stream(gpu_lib, xd, spec.m, k, key_tile=kt, key_partition=kp)
        assert_same(out, ref, f"k={k} key_tile={kt} key_partition={kp}")
    rows = synth.sample_rows(spec, 12, salt=k) + [0, 3, 4, 100]
    rows = sorted(set(r for r in rows if r < spec.S))
    gi = out[0][0].cpu().numpy()[rows]
    gs = out[1][0].cpu().numpy()[rows]
    check_rows(gi, gs, rows, oa["q_bits"], oa["kc_bits"], oa["w"], spec.m, k)


def _structured_keys(kind, T, D=128):
    """Keys whose scores (q = e0, w = 1, one head) are non-decreasing in s
    ('monotone': every key beats the running threshold) or all equal ('constant')."""
    kc = torch.zeros((1, T, D), dtype=torch.float32)
    if kind == "monotone":
        vals = torch.arange(T, dtype=torch.float32) // 4 + 1          # ties in fours
        kc[0, :, 0] = vals
    else:
        kc[0, :, 0] = 1.5
    return kc.to(torch.bfloat16)


@pytest.mark.parametrize("kind,T", [("monotone", 3000), ("constant", 3000), ("monotone", 8192)])
def test_adversarial_orders(gpu_lib, kind, T):
    """T = 8192: rows that see more than 3,584 keys fill their 4096-slot lists, so the
    select stage compacts mid-partition while leaving the final cut to the merge, and
    the merge's keep rule does not fit (every late key lands in the histogram's top
    bin), so its radix fallback runs."""
    S, m, k = 4 * T, 4, 300
    say("adversarial", kind, T)
    q = torch.zeros((1, S, 1, 128), dtype=torch.bfloat16)
    q[..., 0] = 1.0
    w = torch.ones((1, S, 1), dtype=torch.float32)
    kc = _structured_keys(kind, T)
    xd = dev({"q": q, "kc": kc, "w": w})
    ref = run_mat(gpu_lib, xd, m, k)
    for kt in (64, 512):
        assert_same(run_stream(gpu_lib, xd, m, k, key_tile=kt), ref, f"{kind} kt={kt}")
    rows = [0, 3, 1199, 1200, 5000, S - 1]
    if T > 3000:
        rows = [0, 3, 1199, 1200, 14335, 14340, 20000, S - 1]
    oi, ov = oracle.indexer_topk(bits(q), bits(kc), w.numpy(), m, k, rows=rows)
    np.testing.assert_array_equal(ref[0][0].cpu().numpy()[rows], oi[0])
    np.testing.assert_array_equal(ref[1][0].cpu().double().numpy()[rows], ov[0])


# ---------------------------------------------------------------------------
# Small exactness check: duplicates force ties; chunk sweep bit-exact
# ---------------------------------------------------------------------------

def test_small_duplicates_chunk_sweep(gpu_lib):
    spec = synth.CONFIGS["small"]
    say("small", spec)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    ref = run_mat(gpu_lib, xd, spec.m, spec.k)
    for qc in (256, 512, 1024, 2048, 4096):
        for kt in (64, 512, 768, 1024):
            out = run_stream(gpu_lib, xd, spec.m, spec.k, query_chunk=qc, key_tile=kt)
            assert_same(out, ref, f"small query_chunk={qc} key_tile={kt}")
    # ties: each duplicated key scores exactly like its source, the lower index first
    pairs = synth.duplicate_pairs(spec, 0)
    gi, gs = ref[0][0].cpu().numpy(), ref[1][0].cpu().numpy()
    pos = {int(s): j for j, s in enumerate(gi[spec.S - 1]) if s >= 0}
    for s, src in pairs:
        if s in pos and src in pos:
            assert gs[spec.S - 1, pos[s]] == gs[spec.S - 1, pos[src]]
            assert pos[src] < pos[s]
    for b in range(spec.B):
        rows = synth.sample_rows(spec, 24, salt=100 + b)
        check_rows(ref[0][b].cpu().numpy()[rows], ref[1][b].cpu().numpy()[rows], rows,
                   oa["q_bits"], oa["kc_bits"], oa["w"], spec.m, spec.k, b=b)


# ---------------------------------------------------------------------------
# Metamorphic properties and determinism
# ---------------------------------------------------------------------------

def test_metamorphic(gpu_lib):
    spec = synth.InputSpec(B=2, S=1536, T=384, H=64, m=4, k=96, seed=26)
    say("metamorphic")
    xd = dev(synth.make_inputs(spec))
    base = run_stream(gpu_lib, xd, spec.m, spec.k)
    # w x 2: scores double exactly, same indices
    x2 = dict(xd, w=xd["w"] * 2)
    i2, s2 = run_stream(gpu_lib, x2, spec.m, spec.k)
    assert torch.equal(i2, base[0])
    assert torch.equal(s2, base[1] * 2)
    # batch entries are independent: swapping them swaps the outputs
    xs = {"q": xd["q"].flip(0).contiguous(), "kc": xd["kc"].flip(0).contiguous(),
          "w": xd["w"].flip(0).contiguous()}
    fi, fs = run_stream(gpu_lib, xs, spec.m, spec.k)
    assert_same((fi.flip(0), fs.flip(0)), base, "batch swap")
    # a q slice at its absolute offset equals the same rows of the full call
    r0, r1 = 700, 1100
    xsl = {"q": xd["q"][:, r0:r1].contiguous(), "kc": xd["kc"], "w": xd["w"][:, r0:r1].contiguous()}
    si_, ss_ = run_stream(gpu_lib, xsl, spec.m, spec.k, q_pos0=r0)
    assert_same((si_, ss_), (base[0][:, r0:r1], base[1][:, r0:r1]), "q slice")
    # keys beyond every row's view do not matter
    kc2 = xd["kc"].clone()
    kc2[:, 2000 // 4:] = 0
    assert_same(run_stream(gpu_lib, dict(xd, kc=kc2), spec.m, spec.k), base, "late keys")
    # repeated runs are bitwise identical (no races in the selection)
    for _ in range(5):
        assert_same(run_stream(gpu_lib, xd, spec.m, spec.k, key_tile=1024), base, "repeat")


# ---------------------------------------------------------------------------
# Degenerate cases
# ---------------------------------------------------------------------------

def test_degenerate(gpu_lib):
    say("degenerate")
    # no keys at all: every slot is padding
    spec = synth.InputSpec(B=1, S=64, T=0, H=4, m=4, k=8, seed=27)
    x = synth.make_inputs(spec.replace(T=1))
    xd = dev({"q": x["q"], "kc": x["kc"][:, :0].contiguous(), "w": x["w"]})
    gi, gs = run_stream(gpu_lib, xd, 4, 8)
    assert (gi == -1).all() and torch.isneginf(gs).all()
    gi, gs = run_mat(gpu_lib, xd, 4, 8)
    assert (gi == -1).all() and torch.isneginf(gs).all()
    # rows before the first key is visible, k = 1, one head
    spec = synth.InputSpec(B=1, S=40, T=10, H=1, m=4, k=1, seed=28)
    xc = synth.make_inputs(spec)
    xd = dev(xc)
    oa = oracle_args(xc, spec)
    gi, gs = run_stream(gpu_lib, xd, 4, 1)
    check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(40), oa["q_bits"],
               oa["kc_bits"], oa["w"], 4, 1)
    assert (gi[0, :3] == -1).all()
    # S = 0 is a no-op
    e = {"q": xd["q"][:, :0].contiguous(), "kc": xd["kc"], "w": xd["w"][:, :0].contiguous()}
    gi, gs = run_stream(gpu_lib, e, 4, 1)
    assert gi.numel() == 0


def test_errors_raise(gpu_lib):
    spec = synth.InputSpec(B=1, S=64, T=16, H=4, m=4, k=8, seed=29)
    xd = dev(synth.make_inputs(spec))
    with pytest.raises(gpu_lib.SiError, match="UNSUPPORTED"):
        run_stream(gpu_lib, xd, 4, 4096)
    with pytest.raises(gpu_lib.SiError, match="INVALID_ARG"):
        run_stream(gpu_lib, xd, 0, 8)
    with pytest.raises(gpu_lib.SiError, match="UNSUPPORTED"):
        run_stream(gpu_lib, xd, 4, 8, key_tile=100)
    small_ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(gpu_lib.SiError, match="WORKSPACE"):
        gpu_lib.indexer_topk(xd["q"], xd["kc"], xd["w"], 4, 8, ws=small_ws)
