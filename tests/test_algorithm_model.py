"""A plain-Python model of the streaming selection the HIP kernels run (key tiles, a
running threshold, a bounded candidate buffer with exact compaction, key
partitions, a merge of the partition lists), checked on the CPU against the
oracle's stable selection.  It tests the method, independently of the GPU: the
partition-merge identity topk(A u B) = topk(topk(A) u topk(B)) for a strict total
order, and the threshold argument (a key below the k-th of k kept keys can never
enter the top k)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle


def key(score: float, idx: int):
    """Strict total order of the selection: larger score first, then lower index."""
    return (score, -idx)


def stream_partition(scores, lo, hi, k, key_tile, capacity):
    """One (query, partition) of the select kernel: returns its local top-k keys."""
    theta = None                     # running threshold (a key), None = accept all
    buf = []
    for t0 in range(lo, hi, key_tile):
        for s in range(t0, min(t0 + key_tile, hi)):
            kv = key(scores[s], s)
            if theta is None or kv > theta:
                buf.append(kv)
        assert len(buf) <= capacity, "buffer overflow"
        last = t0 + key_tile >= hi
        limit = k if last else capacity - key_tile
        if len(buf) > limit:         # exact compaction: keep the k best, theta = k-th
            buf = sorted(buf, reverse=True)[:k]
            theta = buf[-1]
    return buf


def stream_topk(scores, k, key_tile=512, capacity=2048, partition=None):
    n = len(scores)
    partition = partition or max(n, 1)
    lists = [stream_partition(scores, lo, min(lo + partition, n), k, key_tile, capacity)
             for lo in range(0, n, partition)]
    merged = sorted((kv for lst in lists for kv in lst), reverse=True)[:k]
    idx = [-kv[1] for kv in merged] + [-1] * (k - len(merged))
    return np.asarray(idx, dtype=np.int64)


def rows(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n)
    if kind == "ties":                # few distinct values: massive ties
        return rng.integers(0, 5, n).astype(np.float64)
    if kind == "increasing":          # every key beats the running threshold
        return np.arange(n, dtype=np.float64)
    if kind == "decreasing":
        return -np.arange(n, dtype=np.float64)
    if kind == "constant":
        return np.zeros(n)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "increasing", "decreasing", "constant"])
@pytest.mark.parametrize("n,k,kt,cap,part", [
    (5000, 512, 512, 2048, None), (5000, 512, 64, 2048, 1024), (3000, 1024, 512, 2048, None),
    (9000, 2048, 1024, 4096, 4096), (700, 64, 256, 2048, 256), (100, 512, 512, 2048, None),
    (4096, 1, 128, 2048, 512),
])
def test_stream_model_equals_stable_selection(kind, n, k, kt, cap, part):
    rng = np.random.default_rng(n + k + kt)
    sc = rows(kind, n, rng)
    got = stream_topk(sc, k, kt, cap, part)
    want, _ = oracle.select_topk(sc, k)
    np.testing.assert_array_equal(got, want)


def test_threshold_policy_never_overflows_with_the_planned_capacities():
    """The capacities the planner picks (2048, or 4096 for large k or key tiles)
    leave room for one key tile after every compaction, for every built key tile."""
    for k in (1, 64, 512, 1024, 2048):
        for kt in (64, 128, 256, 512, 768, 1024):
            cap = 2048 if (2 * k <= 2048 and k + kt + 256 <= 2048) else 4096
            assert cap - kt > k           # a compaction always frees room
            sc = np.arange(6 * cap, dtype=np.float64)   # worst case: all keys survive
            stream_topk(sc, k, kt, cap)
