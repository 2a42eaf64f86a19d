"""GPU parity of the low-precision paths: the E4M3 q quantiser and scoring with E4M3 q
against E4M3 keys (row scale) or MXFP4 keys (E8M0 block scales), on the f8f6f4 MFMA.

The quantiser's bytes and weights are compared bit for bit with the oracle's.  Scores
and top-k are compared with the float64 oracle of the quantised operands (the scorer's
own inputs), element by element within the fp32 bound; streaming == materialise bit
for bit under every knob; hand cases exactly.  Recall against the oracle of the
unquantised bf16 q is reported (the quantisation's own effect, not a kernel error)."""

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
KEY_FORMATS = ["e4m3fn", "mxfp4"]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def quantised_inputs(si, spec, x):
    """GPU-quantised q and w_eff, checked bit for bit against the oracle's quantiser;
    returns (device dict with q = E4M3 bytes, w = w_eff; host bits for the oracle)."""
    xd = to_dev(x)
    q8, w_eff, scale = si.quantize_q(xd["q"], xd["w"], with_scale=True)
    torch.cuda.synchronize()
    oq8, ow, osc = oracle.quantize_q_e4m3(bits(x["q"]), x["w"].numpy())
    assert (q8.cpu().numpy() == oq8).all(), "q8 bytes differ from the oracle's"
    assert (w_eff.cpu().numpy().view(np.uint32) == ow.view(np.uint32)).all(), "w_eff bits differ"
    assert (scale.cpu().numpy().view(np.uint32) == osc.view(np.uint32)).all(), "scale bits differ"
    d = {"q": q8, "kc": xd["kc"], "kc_scale": xd["kc_scale"], "w": w_eff}
    host = {"q_bits": oq8, "kc_bits": bits(x["kc"]), "w": ow,
            "kc_scale": None if x["kc_scale"] is None else x["kc_scale"].numpy(),
            "kc_dtype": spec.kc_dtype, "q_dtype": "e4m3fn"}
    return d, host


def stream(si, d, m, k, **kw):
    out = si.indexer_topk(d["q"], d["kc"], d["w"], m, k, kc_scale=d["kc_scale"], **kw)
    torch.cuda.synchronize()
    return out


def mat(si, d, m, k, **kw):
    out = si.materialize_topk(d["q"], d["kc"], d["w"], m, k, kc_scale=d["kc_scale"], **kw)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------

def test_quantize_q_bit_exact_adversarial(gpu_lib):
    """Magnitudes over 10 decades (subnormal and zero codes), an all-zero head, rows whose
    elements land exactly on E4M3 midpoints (ties to even), negative zeros."""
    rnd = np.random.default_rng(11)
    B, S, H, D = 2, 67, 64, 128
    mag = 10.0 ** rnd.uniform(-8, 2, (B, S, H, D))
    q = (rnd.standard_normal((B, S, H, D)) * mag).astype(np.float32)
    q[0, 3, 5] = 0.0
    q[1, 7, 9] = -0.0
    # midpoints: the row maximum 3.5 gives scale 2^-7 exactly; every other element is a
    # midpoint between adjacent E4M3 values, times 2^-7
    vals = oracle.e4m3fn_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2 * 2.0 ** -7
    for (b, s, h) in ((0, 0, 0), (1, 66, 63), (0, 30, 17)):
        row = rnd.choice(mids, D) * rnd.choice([-1, 1], D)
        row[0] = 3.5
        q[b, s, h] = row
    qb = torch.from_numpy(q).to(torch.bfloat16)
    assert (qb[0, 0, 0].float().numpy() == q[0, 0, 0]).all()       # midpoints exact in bf16
    w = torch.from_numpy(rnd.standard_normal((B, S, H)).astype(np.float32))
    spec = synth.InputSpec(B=B, S=S, T=4, H=H, m=4, k=2, kc_dtype="e4m3fn")
    x = {"q": qb, "w": w, "kc": torch.zeros((B, 4, D), dtype=torch.uint8),
         "kc_scale": torch.ones((B, 4))}
    quantised_inputs(gpu_lib, spec, x)


# ---------------------------------------------------------------------------
# Hand cases: every value is exact in E4M3 and in E2M1, so the expected outputs are
# those of the bf16 cases
# ---------------------------------------------------------------------------

def _lowp_case(case, fmt):
    x = build(case)
    q8 = x["q"].float().to(torch.float8_e4m3fn)
    assert torch.equal(q8.float(), x["q"].float()), "hand case q not exact in E4M3"
    if x["kc_dtype"] == "bf16":
        kf = x["kc"].float()
    else:
        kf = x["kc"].view(torch.float8_e4m3fn).float() * x["kc_scale"][..., None]
    if fmt == "e4m3fn":
        kc = kf.to(torch.float8_e4m3fn)
        assert torch.equal(kc.float(), kf)
        kc, ks = kc.view(torch.uint8), torch.ones(kf.shape[:2], dtype=torch.float32)
    else:
        kc, ks = synth.mxfp4_quantize(kf)
        back = oracle.mxfp4_bits_to_f64(kc.numpy(), ks.numpy())
        assert (back == kf.double().numpy()).all(), "hand case keys not exact in MXFP4"
    return {"q": q8.view(torch.uint8), "kc": kc, "kc_scale": ks, "w": x["w"]}, x


@pytest.mark.parametrize("fmt", KEY_FORMATS)
@pytest.mark.parametrize("key_tile", [64, 512])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_lowp_hand_cases_exact(gpu_lib, case, key_tile, fmt):
    say("lowp hand", case["name"], key_tile, fmt)
    d, x = _lowp_case(case, fmt)
    d = to_dev(d)
    eidx, evals = expected(case)
    for out in (stream(gpu_lib, d, x["m"], x["k"], q_pos0=x["q_pos0"], key_tile=key_tile),
                mat(gpu_lib, d, x["m"], x["k"], q_pos0=x["q_pos0"])):
        np.testing.assert_array_equal(out[0].cpu().numpy(), eidx)
        np.testing.assert_array_equal(out[1].cpu().double().numpy(), evals)
        assert not torch.signbit(out[1][out[1] == 0]).any()


def test_lowp_exact_random_codes(gpu_lib):
    """q and key elements drawn from {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4} and weights
    from {+-0.5, +-1}: every product is a multiple of 2^-2 below 16, a 128-term dot stays
    below 2^11 and a head sum over 8 heads below 2^14 with its last bit at 2^-3, so
    every fp32 partial sum is exact and the GPU scores equal the float64 oracle bit for
    bit.  A d-position mismatch between the A and B operands, or a wrong lane layout,
    changes them.  The same keys are exact in MXFP4 too."""
    rnd = np.random.default_rng(5)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, -0.5, -1, -1.5, -2, -3, -4], dtype=np.float32)
    ok = oracle.e4m3fn_encode_rne(vals)
    B, S, T, H, m, k = 1, 160, 160, 8, 1, 24
    q8 = rnd.choice(ok, (B, S, H, 128)).astype(np.uint8)
    k8 = rnd.choice(ok, (B, T, 128)).astype(np.uint8)
    w = rnd.choice([-1.0, -0.5, 0.5, 1.0], (B, S, H)).astype(np.float32)
    ks = np.ones((B, T), dtype=np.float32)
    d = to_dev({"q": torch.from_numpy(q8), "kc": torch.from_numpy(k8),
                "kc_scale": torch.from_numpy(ks), "w": torch.from_numpy(w)})
    sc = gpu_lib.materialize_scores(d["q"], d["kc"], d["w"], m, kc_scale=d["kc_scale"])
    torch.cuda.synchronize()
    ex = oracle.score_rows(q8, k8, w, m, kc_dtype="e4m3fn", kc_scale=ks, q_dtype="e4m3fn")
    g = sc[0].cpu().double().numpy()
    vis = np.isfinite(ex)
    assert (np.isneginf(g) == ~vis).all()
    assert (g[vis] == ex[vis]).all(), f"max diff {np.abs(g[vis] - ex[vis]).max()}"
    # and through the MXFP4 operand: the same key values as E2M1 x 2^e blocks
    kv = oracle.e4m3fn_bits_to_f64(k8)
    packed, scl = synth.mxfp4_quantize(torch.from_numpy(kv.astype(np.float32)))
    assert (oracle.mxfp4_bits_to_f64(packed.numpy(), scl.numpy()) == kv).all()
    d4 = dict(d, kc=packed.to(DEV), kc_scale=scl.to(DEV))
    sc4 = gpu_lib.materialize_scores(d4["q"], d4["kc"], d4["w"], m, kc_scale=d4["kc_scale"])
    torch.cuda.synchronize()
    assert (sc4[0].cpu().double().numpy()[vis] == ex[vis]).all()


# ---------------------------------------------------------------------------
# Every row against the oracle, ragged shapes, knobs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", KEY_FORMATS)
def test_lowp_tiny_every_row(gpu_lib, fmt):
    spec = synth.CONFIGS["tiny"].replace(kc_dtype=fmt)
    say("lowp tiny", fmt)
    x = synth.make_inputs(spec)
    d, h = quantised_inputs(gpu_lib, spec, x)
    gi, gs = stream(gpu_lib, d, spec.m, spec.k)
    st = check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S), h["q_bits"],
                    h["kc_bits"], h["w"], spec.m, spec.k, kc_dtype=fmt, kc_scale=h["kc_scale"],
                    q_dtype="e4m3fn")
    say("lowp tiny", fmt, st)
    assert_same((gi, gs), mat(gpu_lib, d, spec.m, spec.k), f"{fmt} tiny stream vs materialise")
    sc = gpu_lib.materialize_scores(d["q"], d["kc"], d["w"], spec.m, kc_scale=d["kc_scale"])
    torch.cuda.synchronize()
    check_score_block(sc[0].cpu().numpy(), range(spec.S), h["q_bits"], h["kc_bits"], h["w"],
                      spec.m, kc_dtype=fmt, kc_scale=h["kc_scale"], q_dtype="e4m3fn")
    # recall against the unquantised bf16 q (the quantisation's effect), reported
    oi, _ = oracle.indexer_topk(bits(x["q"]), h["kc_bits"], x["w"].numpy(), spec.m, spec.k,
                                kc_dtype=fmt, kc_scale=h["kc_scale"])
    g = gi[0].cpu().numpy()
    rec = []
    for t in range(spec.S):
        n = min(spec.k, oracle.visible_count(t, spec.m, spec.T))
        if n:
            rec.append(len(set(g[t, :n]) & set(oi[0, t, :n])) / n)
    say(f"lowp tiny {fmt}: recall vs the bf16-q oracle mean {np.mean(rec):.4f} min {np.min(rec):.4f}")
    assert np.mean(rec) > 0.5


@pytest.mark.parametrize("fmt", KEY_FORMATS)
@pytest.mark.parametrize("q_pos0", [0, 37])
def test_lowp_ragged_every_row(gpu_lib, fmt, q_pos0):
    spec = synth.InputSpec(B=2, S=1000, T=250, H=64, m=4, k=64, seed=21, kc_dtype=fmt)
    say("lowp ragged", fmt, q_pos0)
    x = synth.make_inputs(spec)
    d, h = quantised_inputs(gpu_lib, spec, x)
    gi, gs = stream(gpu_lib, d, spec.m, spec.k, q_pos0=q_pos0)
    for b in range(spec.B):
        check_rows(gi[b].cpu().numpy(), gs[b].cpu().numpy(), range(spec.S), h["q_bits"],
                   h["kc_bits"], h["w"], spec.m, spec.k, q_pos0=q_pos0, b=b, kc_dtype=fmt,
                   kc_scale=h["kc_scale"], q_dtype="e4m3fn")
    assert_same((gi, gs), mat(gpu_lib, d, spec.m, spec.k, q_pos0=q_pos0), f"{fmt} ragged")


@pytest.mark.parametrize("fmt", KEY_FORMATS)
@pytest.mark.parametrize("H,S,key_tile", [(3, 300, 512), (13, 700, 64), (128, 700, 1024)])
def test_lowp_odd_heads(gpu_lib, fmt, H, S, key_tile):
    spec = synth.InputSpec(B=1, S=S, T=S, H=H, m=1, k=100, seed=22 + H, kc_dtype=fmt)
    say("lowp odd heads", fmt, H, S, key_tile)
    x = synth.make_inputs(spec)
    d, h = quantised_inputs(gpu_lib, spec, x)
    gi, gs = stream(gpu_lib, d, spec.m, spec.k, key_tile=key_tile)
    check_rows(gi[0].cpu().numpy(), gs[0].cpu().numpy(), range(spec.S), h["q_bits"],
               h["kc_bits"], h["w"], spec.m, spec.k, kc_dtype=fmt, kc_scale=h["kc_scale"],
               q_dtype="e4m3fn")
    assert_same((gi, gs), mat(gpu_lib, d, spec.m, spec.k), f"{fmt} odd heads")


@pytest.mark.parametrize("fmt", KEY_FORMATS)
def test_lowp_knobs_bit_identical(gpu_lib, fmt):
    """Every key tile, query chunk and key partition gives the same bits, equal to the
    materialise path (two batch entries with 5% duplicate keys: ties)."""
    spec = synth.CONFIGS["small"].replace(S=4096, T=1024, k=256, kc_dtype=fmt)
    say("lowp knobs", fmt)
    x = synth.make_inputs(spec, device=DEV)
    q8, w_eff = gpu_lib.quantize_q(x["q"], x["w"])
    d = {"q": q8, "kc": x["kc"], "kc_scale": x["kc_scale"], "w": w_eff}
    base = mat(gpu_lib, d, spec.m, spec.k, row_block=1024)
    for kt in (64, 128, 256, 512, 768, 1024):
        assert_same(stream(gpu_lib, d, spec.m, spec.k, key_tile=kt), base, f"{fmt} key_tile {kt}")
    for qc in (256, 1000, 4096):
        assert_same(stream(gpu_lib, d, spec.m, spec.k, query_chunk=qc), base, f"{fmt} chunk {qc}")
    assert_same(stream(gpu_lib, d, spec.m, spec.k, key_tile=256, key_partition=256), base,
                f"{fmt} partitions")
    for k in (1, 700, 2048):
        assert_same(stream(gpu_lib, d, spec.m, k), mat(gpu_lib, d, spec.m, k, row_block=1024),
                    f"{fmt} k={k}")


def test_lowp_rejects_unbuilt_pairs(gpu_lib):
    from streaming_top_selection_amd import SiError
    spec = synth.CONFIGS["tiny"].replace(S=64, T=16, H=4)
    x = to_dev(synth.make_inputs(spec))
    q8, w_eff = gpu_lib.quantize_q(x["q"], x["w"])
    with pytest.raises(SiError, match="E4M3 q takes"):
        gpu_lib.indexer_topk(q8, x["kc"], w_eff, 4, 8)                  # bf16 keys
    kc4, ks4 = synth.mxfp4_quantize(x["kc"].float().cpu())
    with pytest.raises(SiError, match="MXFP4 keys need E4M3 q"):
        gpu_lib.indexer_topk(x["q"], kc4.to(DEV), x["w"], 4, 8, kc_scale=ks4.to(DEV))
