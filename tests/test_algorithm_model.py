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


def ord32(x: float) -> int:
    """Order-preserving 32-bit image of a float32 (the upper half of a selection key)."""
    u = int(np.float32(x).view(np.uint32))
    return (~u & 0xFFFFFFFF) if u & 0x80000000 else (u | 0x80000000)


def key64(score: float, idx: int) -> int:
    return (ord32(score) << 32) | (~idx & 0xFFFFFFFF)


def compact_model(keys, k, keep_max):
    """The kernel's compaction threshold: 256 bins linear in the score image between the
    smallest and the largest key (integer arithmetic as on the GPU); keep the bin holding
    the k-th key whole if that stays within keep_max, else rank that bin's keys exactly.
    Returns the kept keys (all keys >= the smallest kept one)."""
    keys = sorted(keys, reverse=True)
    imgs = [kk >> 32 for kk in keys]
    omin, omax = min(imgs), max(imgs)
    if omax > omin:
        mul = (256 << 32) // (omax - omin + 1)
        bins = [min(255, ((o - omin) * mul) >> 32) for o in imgs]
        d = bins[k - 1]                       # bin of the k-th largest (keys sorted)
        above = sum(1 for b in bins if b > d)
        cnt = sum(1 for b in bins if b == d)
        if above + cnt <= keep_max:
            return [kk for kk, b in zip(keys, bins) if b >= d]
    return keys[:k]                           # exact: the k-th key as threshold


def stream_partition(scores, lo, hi, k, key_tile, capacity, keep_mid=None):
    """One (query, partition) of the select kernel: returns its kept keys.  The filter
    compares scores only (a key seen later has a larger index than the threshold key,
    so an equal score never passes); mid-partition compactions keep between k and
    keep_mid keys, the last one exactly k."""
    keep_mid = k if keep_mid is None else keep_mid
    thf = -np.inf                      # running threshold score
    buf = []
    for t0 in range(lo, hi, key_tile):
        for s in range(t0, min(t0 + key_tile, hi)):
            if scores[s] > thf:
                buf.append(key64(scores[s], s))
        assert len(buf) <= capacity, "buffer overflow"
        last = t0 + key_tile >= hi
        limit = k if last else capacity - key_tile
        if len(buf) > limit:
            buf = compact_model(buf, k, k if last else keep_mid)
            assert k <= len(buf) <= (k if last else keep_mid)
            lowest = min(buf) >> 32
            thf = float(np.array([lowest ^ 0x80000000 if lowest & 0x80000000 else ~lowest & 0xFFFFFFFF],
                                 dtype=np.uint32).view(np.float32)[0])
    return buf


def stream_topk(scores, k, key_tile=512, capacity=2048, partition=None, keep_mid=None):
    n = len(scores)
    partition = partition or max(n, 1)
    lists = [stream_partition(scores, lo, min(lo + partition, n), k, key_tile, capacity, keep_mid)
             for lo in range(0, n, partition)]
    merged = sorted((kk for lst in lists for kk in lst), reverse=True)[:k]
    idx = [~(kk & 0xFFFFFFFF) & 0xFFFFFFFF for kk in merged] + [-1] * (k - len(merged))
    return np.asarray(idx, dtype=np.int64)


def rows(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32).astype(np.float64)
    if kind == "ties":                # few distinct values: massive ties
        return rng.integers(0, 5, n).astype(np.float64)
    if kind == "close":               # distinct scores within a few ulps: one bin
        return (1.0 + rng.integers(0, 40, n) * 2.0 ** -23)
    if kind == "increasing":          # every key beats the running threshold
        return np.arange(n, dtype=np.float64)
    if kind == "decreasing":
        return -np.arange(n, dtype=np.float64)
    if kind == "constant":
        return np.zeros(n)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "increasing", "decreasing", "constant",
                                  "close"])
@pytest.mark.parametrize("n,k,kt,cap,part", [
    (5000, 512, 512, 2048, None), (5000, 512, 64, 2048, 1024), (3000, 1024, 512, 2048, None),
    (9000, 2048, 1024, 4096, 4096), (700, 64, 256, 2048, 256), (100, 512, 512, 2048, None),
    (4096, 1, 128, 2048, 512),
])
def test_stream_model_equals_stable_selection(kind, n, k, kt, cap, part):
    rng = np.random.default_rng(n + k + kt)
    sc = rows(kind, n, rng)
    want, _ = oracle.select_topk(sc, k)
    # the kernel's policy: mid-partition compactions keep up to k + a quarter of the room
    keep_mid = k + (cap - kt - k) // 4
    np.testing.assert_array_equal(stream_topk(sc, k, kt, cap, part, keep_mid), want)
    np.testing.assert_array_equal(stream_topk(sc, k, kt, cap, part, k), want)


@pytest.mark.parametrize("kind", ["normal", "ties", "constant", "close", "increasing"])
@pytest.mark.parametrize("cnt,k,keep_max", [(2000, 512, 512), (2000, 512, 768), (600, 512, 512),
                                             (1537, 1, 1), (4000, 2048, 2560)])
def test_compaction_keeps_a_top_prefix(kind, cnt, k, keep_max):
    """The compaction's kept set is exactly the |kept| largest keys, k <= |kept| <=
    keep_max (exactly k when keep_max == k)."""
    rng = np.random.default_rng(cnt + k)
    sc = rows(kind, cnt, rng)
    keys = [key64(float(v), i) for i, v in enumerate(sc)]
    kept = compact_model(keys, k, keep_max)
    assert k <= len(kept) <= keep_max
    assert sorted(kept, reverse=True) == sorted(keys, reverse=True)[:len(kept)]


def test_threshold_policy_never_overflows_with_the_planned_capacities():
    """The capacities the planner picks (2048, or 4096 for large k or key tiles)
    leave room for one key tile after every compaction, for every built key tile."""
    for k in (1, 64, 512, 1024, 2048):
        for kt in (64, 128, 256, 512, 768, 1024):
            cap = 2048 if (2 * k <= 2048 and k + kt + 256 <= 2048) else 4096
            assert cap - kt > k           # a compaction always frees room
            sc = np.arange(6 * cap, dtype=np.float64)   # worst case: all keys survive
            stream_topk(sc, k, kt, cap)
