"""Builds the inputs of the hand cases in ``tests/golden/hand_cases.json``."""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _dense(sparse: dict, D: int) -> np.ndarray:
    v = np.zeros(D, dtype=np.float32)
    for dim, val in sparse.items():
        v[int(dim)] = val
    return v


def build(case):
    """Inputs of one case: dict(q bf16 [1,S,H,D], kc, kc_scale, w [1,S,H], m, k, q_pos0,
    kc_dtype) as CPU torch tensors."""
    S, H, D, T = case["S"], case["H"], case["D"], case["T"]
    q = np.zeros((1, S, H, D), dtype=np.float32)
    rows = case["q"]
    for t in range(S):
        heads = rows[0] if case.get("q_same_for_all_rows") else rows[t]
        for h in range(H):
            q[0, t, h] = _dense(heads[h], D)
    w = np.tile(np.asarray(case["w"], dtype=np.float32), (1, S, 1))
    kc_dtype = case.get("kc_dtype", "bf16")
    if kc_dtype == "bf16":
        kc = torch.from_numpy(np.stack([_dense(k, D) for k in case["keys"]])[None]
                              ).to(torch.bfloat16)
        kc_scale = None
    else:
        raw = np.zeros((1, T, D), dtype=np.uint8)
        for s, sparse in enumerate(case["keys_e4m3_bytes"]):
            for dim, byte in sparse.items():
                raw[0, s, int(dim)] = byte
        kc = torch.from_numpy(raw)
        kc_scale = torch.tensor([case["kc_scale"]], dtype=torch.float32)
    return {
        "q": torch.from_numpy(q).to(torch.bfloat16),
        "kc": kc,
        "kc_scale": kc_scale,
        "w": torch.from_numpy(w),
        "m": case["m"],
        "k": case["k"],
        "q_pos0": case["q_pos0"],
        "kc_dtype": kc_dtype,
    }


def expected(case):
    idx = np.asarray(case["expect_idx"], dtype=np.int64)[None]
    val = np.asarray([[(-math.inf if v == "-inf" else float(v)) for v in row]
                      for row in case["expect_score"]], dtype=np.float64)[None]
    return idx, val


def bits(x: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16 (as uint16) or E4M3 (uint8) tensor, as a numpy array."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.uint8:
        return x.numpy()
    raise TypeError(x.dtype)
