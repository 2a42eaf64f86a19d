"""si_indexer_topk_noalloc (static scratch, no allocation) against si_indexer_topk with
a caller workspace, through the C ABI: bit-identical outputs on two calls in a row,
the second one smaller, and a clear error for a problem that does not fit."""

from __future__ import annotations

import ctypes
import sys

import pytest
import torch

import synth
from parity import assert_same

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def noalloc(lib, x, spec, k, q_pos0=0, query_chunk=0):
    """Calls si_indexer_topk_noalloc through ctypes; returns (status, (idx, score))."""
    from streaming_top_selection_amd import _lib
    q, kc, w, ks = x["q"], x["kc"], x["w"], x["kc_scale"]
    B, S, H, D = q.shape
    T = kc.shape[1]
    out = (torch.full((B, S, k), 7, dtype=torch.int32, device=DEV),
           torch.full((B, S, k), 7.0, dtype=torch.float32, device=DEV))
    cfg = _lib.SiConfig(0, query_chunk, 0, 0)
    kcd = _lib.SI_BF16 if ks is None else _lib.SI_FP8_E4M3FN
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())   # noqa: E731
    st = lib.si_indexer_topk_noalloc(
        ptr(q), _lib.SI_BF16, ptr(kc), kcd, ptr(ks), ptr(w), B, S, T, H, D, spec.m, k, q_pos0,
        ctypes.byref(cfg), ptr(out[0]), ptr(out[1]),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, out


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    from streaming_top_selection_amd import _lib
    lib = _lib.load()
    # first call: two batch entries, 5% duplicate keys (ties), several query chunks (its
    # workspace at one chunk would be 277 MB, more than the 256 MiB scratch)
    big = synth.CONFIGS["small"]
    pl = gpu_lib.plan(big.B, big.S, big.T, big.H, big.D, big.m, big.k)
    assert pl.workspace_bytes > _lib.SI_NOALLOC_SCRATCH_BYTES
    say("noalloc big", big)
    xb = synth.make_inputs(big, device=DEV)
    st, out = noalloc(lib, xb, big, big.k)
    assert st == _lib.SI_OK, lib.si_last_error()
    ref = gpu_lib.indexer_topk(xb["q"], xb["kc"], xb["w"], big.m, big.k)
    torch.cuda.synchronize()
    assert_same(out, ref, "noalloc big")
    del xb, out, ref
    # second call: smaller, ragged, E4M3 keys with a row scale, a q offset
    small = synth.InputSpec(B=1, S=1000, T=250, H=64, m=4, k=64, seed=23, kc_dtype="e4m3fn")
    say("noalloc small", small)
    xs = synth.make_inputs(small, device=DEV)
    st, out = noalloc(lib, xs, small, small.k, q_pos0=37)
    assert st == _lib.SI_OK, lib.si_last_error()
    ref = gpu_lib.indexer_topk(xs["q"], xs["kc"], xs["w"], small.m, small.k,
                               kc_scale=xs["kc_scale"], q_pos0=37)
    torch.cuda.synchronize()
    assert_same(out, ref, "noalloc small")


def test_noalloc_rejects_what_does_not_fit(gpu_lib):
    from streaming_top_selection_amd import _lib
    lib = _lib.load()
    spec = synth.CONFIGS["small"]
    x = synth.make_inputs(spec, device=DEV)
    # one query chunk of all 8192 rows x 2 batch entries needs 277 MB of workspace
    st, out = noalloc(lib, x, spec, spec.k, query_chunk=8192)
    assert st == _lib.SI_ERR_WORKSPACE
    assert b"static scratch" in lib.si_last_error()
    # nothing was written
    assert (out[0] == 7).all().item()
