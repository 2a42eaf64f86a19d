"""Benchmark of the lightning-indexer top-k step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v4flash]

A step is one pass of the whole hot path over the workload: for every query chunk,
the fused score + select kernel and then the merge kernel (exactly what
si_indexer_topk enqueues).  Inputs are synthetic, drawn on the GPU before the timed
region.  Prints one JSON line:

  value      scored (query, key) pairs per second: causally visible pairs / step time
  roofline   the fused select kernel: algorithmic MFMA flops per launch (visible pairs
             x 2 H D) / its mean launch duration (HIP events on the launch stream),
             against the bf16 dense MFMA peak
  merge      algorithmic bytes of the merge kernel / its mean duration vs 8 TB/s
  peak HBM   torch's allocator peak (inputs + outputs + workspace)
  cpu_baseline  the float64 CPU oracle on a bounded sample of query rows of the same
             workload, in the same pairs/s unit
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

METRIC = "indexer scored q·k pairs/s + peak HBM at S=64K V4-Flash; % MFMA peak"
BF16_DENSE_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP8_DENSE_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (the f8f6f4 ops on E4M3)
HBM_PEAK_GBPS = 8000.0              # MI355X HBM3E

WORKLOADS = {
    "v4flash": "V4-Flash indexer layer: B=1, S=65536 queries, m=4, T=16384 compressed keys, "
               "H_I=64, D=128, top-k=512, bf16 q/k with per-channel U(0.5,2) scales, "
               "fp32 w ~ N(0,1)/8, causal",
    "tiny": "Tiny indexer: B=1, S=1024, m=4, T=256, H_I=64, D=128, top-k=64",
    "small": "Small exactness check: B=2, S=8192, m=4, T=2048, H_I=64, D=128, top-k=512, 5% duplicate keys",
    "long": "Long-context: B=1, S=262144, m=4, T=65536, H_I=64, D=128, top-k=512, bf16 q/k",
    "million": "Million-token capacity: B=1, S=1048576, m=4, T=262144, H_I=64, D=128, top-k=512, "
               "bf16 q, E4M3 keys with per-row fp32 scale",
    "v4flash-fp8": "V4-Flash indexer layer with fp8 operands: B=1, S=65536, m=4, T=16384, H_I=64, "
                   "D=128, top-k=512; q quantised per (row, head) to E4M3 inside the step (scale "
                   "folded into w), keys E4M3 with per-row fp32 scale (per-channel U(0.5,2) data), "
                   "f8f6f4 MFMA",
    "v4flash-mxfp4": "V4-Flash indexer layer with MXFP4 keys: B=1, S=65536, m=4, T=16384, H_I=64, "
                     "D=128, top-k=512; q quantised per (row, head) to E4M3 inside the step, keys "
                     "MXFP4 (E2M1 + E8M0 per 32), scaled f8f6f4 MFMA",
}
WORKLOADS["long-two-stage"] = (
    "Two-stage indexer at the long-context shape: B=1, S=262144, m=4, T=65536, H_I=64, D=128; "
    "block keys = bf16 mean of 8 keys, coarse top-2048 blocks, fine top-512 of their keys "
    "(+ the trailing incomplete block), bf16")
WORKLOADS["million-bf16"] = (
    "Million-token shape with bf16 keys: B=1, S=1048576, m=4, T=262144, H_I=64, D=128, "
    "top-k=512, bf16 q/k (the single-stage reference for million-two-stage)")
WORKLOADS["million-two-stage"] = (
    "Two-stage indexer at the million-token shape: B=1, S=1048576, m=4, T=262144, H_I=64, "
    "D=128; block keys = bf16 mean of 8 keys, coarse top-2048 blocks, fine top-512 of their "
    "keys (+ the trailing incomplete block), bf16")
TWO_STAGE = {"long-two-stage": dict(block=8, k_blocks=2048),
             "million-two-stage": dict(block=8, k_blocks=2048)}
WORKLOADS["compose-long"] = (
    "Indexer composed with the sparse-attention consumer at the long-context shape: B=1, "
    "S=262144, m=4, T=65536, H_I=64, D=128, top-k=512 (streaming indexer), then softmax "
    "attention of 64 heads over the 512 selected compressed latents (key = value, D=128), "
    "bf16")
COMPOSE = {"compose-long": dict(HA=64)}
# workload -> input configuration (synth.CONFIGS); the fp8-q workloads quantise q in the step
WORKLOAD_SPEC = {"v4flash-fp8": "v4flash-e4m3", "v4flash-mxfp4": "v4flash-mxfp4",
                 "long-two-stage": "long", "compose-long": "long",
                 "million-two-stage": "million-bf16"}
FP8_Q = {"v4flash-fp8", "v4flash-mxfp4"}
DTYPE_NAME = {("bf16", "bf16"): "bf16", ("bf16", "e4m3fn"): "bf16",
              ("e4m3fn", "e4m3fn"): "e4m3", ("e4m3fn", "mxfp4"): "e4m3xe2m1"}
# default (steps, warmup) per workload: about a minute of timed work at most
DEFAULT_STEPS = {"long": (5, 1), "million": (3, 1), "long-two-stage": (5, 1),
                 "compose-long": (5, 1), "million-bf16": (3, 1), "million-two-stage": (3, 1)}
# q rows per slice of the million workload's streamed-q capacity pass
CAPACITY_SLICE_ROWS = 16384


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["si_select.hpp", "si_select_inst.hip", "si_compact.hpp", "si_score.hpp",
                  "si_score_q8.hpp", "si_common.hpp"]
PROFILE_SUMMARY = {"v4flash": os.path.join(ROOT, "profiles", "select_kernel_v4flash_s65536.md"),
                   "v4flash-fp8": os.path.join(ROOT, "profiles",
                                               "select_kernel_v4flash_fp8_s65536.md")}
COPY_PROBE_BYTES = 1 << 30


def kernel_source_hash():
    """SHA-256 (first 16 hex digits) of the fused select kernel's sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "streaming_top_selection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload="v4flash"):
    """HBM bytes per select launch from the committed counter summary of the workload,
    if it was taken on the current kernel sources (else None: the counters no longer
    apply)."""
    try:
        text = open(PROFILE_SUMMARY[workload]).read()
    except (OSError, KeyError):
        return None
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


def visible_pairs(S, T, m, q_pos0=0):
    """Sum over rows of min(T, (q_pos0 + t + 1) // m), in closed form per segment."""
    import numpy as np
    t = np.arange(q_pos0, q_pos0 + S, dtype=np.int64)
    return int(np.minimum(T, (t + 1) // m).sum())


def two_stage_pairs(S, T, m, block, k_blocks, q_pos0=0):
    """(coarse pairs, fine pairs) summed over rows: the complete visible blocks each
    query scores, and its fine candidates (kept blocks' keys + trailing keys)."""
    import numpy as np
    t = np.arange(q_pos0, q_pos0 + S, dtype=np.int64)
    n = np.minimum(T, (t + 1) // m)
    nb = np.minimum(T // block, (t + 1) // (block * m))
    fine = block * np.minimum(nb, k_blocks) + (n - block * nb)
    return int(nb.sum()), int(fine.sum())


def bench_two_stage(args, spec, dev):
    """One step = block keys + the two-stage top-k over every query row (what
    si_block_keys_mean + si_indexer_topk_two_stage enqueue), inputs resident."""
    import numpy as np
    import torch

    import streaming_top_selection_amd as si
    import synth
    ts = TWO_STAGE[args.workload]
    x = synth.make_inputs(spec, device=dev)
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    input_bytes = tensor_bytes(x["q"], x["kc"], x["w"])
    kb = torch.empty((spec.B, spec.T // ts["block"], spec.D), dtype=torch.bfloat16, device=dev)
    pl = si.two_stage_plan(spec.B, spec.S, spec.T, spec.H, spec.D, spec.m, spec.k,
                           ts["k_blocks"], ts["block"], query_chunk=args.query_chunk)
    ws = torch.empty(max(pl.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    out = (torch.empty((spec.B, spec.S, spec.k), dtype=torch.int32, device=dev),
           torch.empty((spec.B, spec.S, spec.k), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def step():
        si.block_keys(x["kc"], ts["block"], out=kb)
        si.indexer_topk_two_stage(x["q"], x["kc"], kb, x["w"], spec.m, spec.k,
                                  k_blocks=ts["k_blocks"], block=ts["block"],
                                  query_chunk=args.query_chunk, out=out, ws=ws)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_s = wall / args.steps
    ev_s = sum(a.elapsed_time(b) for a, b in evs) / len(evs) / 1e3
    peak = torch.cuda.max_memory_allocated(dev)
    vis = spec.B * visible_pairs(spec.S, spec.T, spec.m)
    cp, fp = two_stage_pairs(spec.S, spec.T, spec.m, ts["block"], ts["k_blocks"])
    flops = spec.B * (cp + fp) * 2 * spec.H * spec.D
    tflops = flops / ev_s / 1e12
    rec = {
        "metric": METRIC, "value": vis / step_s, "unit": "pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "B": spec.B, "S": spec.S, "T": spec.T,
                   "H_I": spec.H, "D": spec.D, "m": spec.m, "k": spec.k,
                   "block": ts["block"], "k_blocks": ts["k_blocks"],
                   "query_chunk": pl.query_chunk, "n_chunks": pl.n_chunks},
        "value_note": "value = causally visible (query, key) pairs of the single-stage problem "
                      "per second; the two stages score scored_pairs of them",
        "visible_pairs": vis,
        "scored_pairs": {"coarse_block_pairs": spec.B * cp, "fine_candidate_pairs": spec.B * fp},
        "peak_hbm_bytes": int(peak), "peak_hbm_gib": peak / 2 ** 30,
        "hbm_bytes": {"inputs": input_bytes, "outputs": tensor_bytes(*out),
                      "block_keys": tensor_bytes(kb), "workspace": int(ws.numel())},
        "roofline": {
            "kernel": "two-stage path (coarse select + merge, fine score, fine select; one call)",
            "bound": "mfma", "achieved": tflops, "peak": BF16_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / BF16_DENSE_PEAK_TFLOPS, "traffic": None,
            "mean_launch_ms": ev_s * 1e3, "flops_per_step": flops},
    }
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        import oracle
        rows = synth.sample_rows(spec.replace(k=8 * ts["k_blocks"]), 4096, salt=100)
        rng = np.random.default_rng(100)
        rng.shuffle(rows)
        kcb = x["kc"][0:1].cpu().view(torch.int16).numpy().view(np.uint16)
        done, pairs, hits = 0.0, 0, []
        got = out[0][0].cpu().numpy()
        while rows and done < args.cpu_seconds:
            r = rows.pop()
            qb = x["q"][0:1, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
            wb = x["w"][0:1, r:r + 1].cpu().numpy()
            t1 = time.perf_counter()
            oi, _ = oracle.two_stage_topk(qb, kcb, wb, spec.m, spec.k, k_blocks=ts["k_blocks"],
                                          block=ts["block"], q_pos0=r)
            done += time.perf_counter() - t1
            pairs += visible_pairs(1, spec.T, spec.m, q_pos0=r)
            o = set(oi[0, 0].tolist()) - {-1}
            hits.append(len(set(got[r].tolist()) & o) / max(1, len(o)))
        rec["cpu_baseline"] = {
            "value": pairs / done if done > 0 else 0.0, "unit": "pairs/s",
            "cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model_name(),
            "kind": "oracle",
            "sample": f"{len(hits)} query rows that see > 2048 complete blocks, the float64 "
                      f"two-stage oracle, {pairs} visible pairs in {done:.1f} s"}
        rec["oracle_sample_recall"] = {"rows": len(hits), "mean": float(np.mean(hits)),
                                       "min": float(np.min(hits))}
    print(json.dumps(rec), flush=True)
    return 0


def bench_compose(args, spec, dev):
    """One step = the streaming indexer top-k (si_indexer_topk) then the sparse attention
    over its selection (si_sparse_attention), inputs resident."""
    import numpy as np
    import torch

    import streaming_top_selection_amd as si
    import synth
    HA = COMPOSE[args.workload]["HA"]
    x = synth.make_inputs(spec, device=dev)
    qa, kv = synth.gen_attention_inputs(spec, HA, device=dev)
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    input_bytes = tensor_bytes(x["q"], x["kc"], x["w"], qa, kv)
    pl = si.plan(spec.B, spec.S, spec.T, spec.H, spec.D, spec.m, spec.k)
    ws = si.workspace(pl, dev)
    sel = (torch.empty((spec.B, spec.S, spec.k), dtype=torch.int32, device=dev),
           torch.empty((spec.B, spec.S, spec.k), dtype=torch.float32, device=dev))
    o = torch.empty((spec.B, spec.S, HA, spec.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        si.indexer_topk(x["q"], x["kc"], x["w"], spec.m, spec.k, out=sel, ws=ws)
        if ev:
            ev[1].record(stream)
        si.sparse_attention(qa, kv, sel[0], out=o)
        if ev:
            ev[2].record(stream)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_s = wall / args.steps
    ix_s = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs) / 1e3
    at_s = sum(e[1].elapsed_time(e[2]) for e in evs) / len(evs) / 1e3
    peak = torch.cuda.max_memory_allocated(dev)
    vis = spec.B * visible_pairs(spec.S, spec.T, spec.m)
    t = np.arange(spec.S, dtype=np.int64)
    nsel = int(np.minimum(spec.k, np.minimum(spec.T, (t + 1) // spec.m)).sum()) * spec.B
    at_flops = nsel * HA * spec.D * 4              # score and value products, 2 flop each
    ix_flops = vis * 2 * spec.H * spec.D
    rec = {
        "metric": METRIC, "value": vis / step_s, "unit": "pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "B": spec.B, "S": spec.S, "T": spec.T,
                   "H_I": spec.H, "D": spec.D, "m": spec.m, "k": spec.k, "H_A": HA},
        "value_note": "value = the indexer's causally visible pairs per second of the whole "
                      "composed step (indexer + attention)",
        "indexer_ms": ix_s * 1e3, "attention_ms": at_s * 1e3,
        "peak_hbm_bytes": int(peak), "peak_hbm_gb": peak / 1e9,
        "hbm_bytes": {"inputs": input_bytes, "selection": tensor_bytes(*sel),
                      "attention_out": tensor_bytes(o), "workspace": int(ws.numel())},
        "roofline": {
            "kernel": "select_kernel (fused bf16 MFMA scoring + running top-k), the indexer "
                      "stage of the step",
            "bound": "mfma", "achieved": ix_flops / ix_s / 1e12, "peak": BF16_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": ix_flops / ix_s / 1e12 / BF16_DENSE_PEAK_TFLOPS,
            "traffic": None, "mean_launch_ms": ix_s * 1e3, "flops_per_step": ix_flops},
        "attention": {
            "kernel": "sparse_attention_kernel (gathered latents, bf16 MFMA, online softmax)",
            "bound": "mfma", "achieved": at_flops / at_s / 1e12, "peak": BF16_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": at_flops / at_s / 1e12 / BF16_DENSE_PEAK_TFLOPS,
            "gathered_bytes": nsel * spec.D * 2,
            "gather_gbps": nsel * spec.D * 2 / at_s / 1e9},
    }
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        import oracle
        rows = synth.sample_rows(spec, 4096, salt=100)
        np.random.default_rng(100).shuffle(rows)
        kcb = x["kc"].cpu().view(torch.int16).numpy().view(np.uint16)
        kvb = kv.cpu().view(torch.int16).numpy().view(np.uint16)
        done, pairs, n = 0.0, 0, 0
        while rows and done < args.cpu_seconds:
            r = rows.pop()
            qb = x["q"][:, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
            qab = qa[:, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
            t1 = time.perf_counter()
            oi, _ = oracle.indexer_topk(qb, kcb, x["w"][:, r:r + 1].cpu().numpy(), spec.m, spec.k,
                                        q_pos0=r)
            oracle.sparse_attention(qab, kvb, oi, oracle.default_scale(spec.D))
            done += time.perf_counter() - t1
            pairs += visible_pairs(1, spec.T, spec.m, q_pos0=r)
            n += 1
        rec["cpu_baseline"] = {
            "value": pairs / done if done > 0 else 0.0, "unit": "pairs/s",
            "cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model_name(),
            "kind": "oracle",
            "sample": f"{n} query rows, float64 oracle indexer + attention, {pairs} visible "
                      f"pairs in {done:.1f} s"}
    print(json.dumps(rec), flush=True)
    return 0


def gemm_ceiling():
    """The dense bf16 MFMA rate a library GEMM (torch -> hipBLASLt) reaches on this GPU,
    square n x n x n products of N(0,1) data: the practical ceiling the select kernel's
    fraction of the nominal peak is read against."""
    import torch
    dev = torch.device("cuda", 0)
    rec = {}
    for n in (4096, 8192, 16384):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            a @ b
        torch.cuda.synchronize(dev)
        reps = 20 if n < 16384 else 6
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            a @ b
        e1.record()
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1) / reps
        tf = 2 * n ** 3 / ms / 1e9
        rec[str(n)] = {"ms": ms, "tflops": tf, "frac_of_bf16_peak": tf / BF16_DENSE_PEAK_TFLOPS}
    print(json.dumps({"gemm_ceiling_bf16": rec}), flush=True)
    return 0


def list_lengths(si, spec, pl, ws, qop, x, knobs):
    """Keys the select stage leaves in the lists of every query row (summed over the
    query chunks: one more select launch per chunk, each list count read back)."""
    import numpy as np
    import torch
    nrows_ws = spec.B * pl.query_chunk * pl.n_partitions
    cand_bytes = -(-nrows_ws * (pl.cand_capacity + 64) * 8 // 256) * 256
    total = 0
    for c in range(pl.n_chunks):
        si.indexer_select_chunk(qop[0], x["kc"], qop[1], spec.m, spec.k, c, ws,
                                kc_scale=x["kc_scale"], **knobs)
        torch.cuda.synchronize()
        rows = min(spec.S, (c + 1) * pl.query_chunk) - c * pl.query_chunk
        cnt = ws[cand_bytes:cand_bytes + nrows_ws * 4].view(torch.int32).cpu().numpy()
        cnt = cnt.reshape(spec.B, pl.query_chunk, pl.n_partitions)[:, :rows]
        total += int(np.minimum(np.maximum(cnt, 0), pl.cand_capacity).sum())
    return total


def cpu_model_name():
    """The host CPU's model name (lscpu), or /proc/cpuinfo's, or "unknown"."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def tensor_bytes(*ts):
    return int(sum(t.numel() * t.element_size() for t in ts if t is not None))


def capacity_pass(si, spec, kc, kc_scale, w, dev, slice_rows=CAPACITY_SLICE_ROWS):
    """The million-token run with q never resident whole: each slice of q rows is drawn,
    scored at its absolute offset (q_pos0) into its rows of the outputs, then freed.
    Returns (allocator peak over the pass, seconds of indexer calls, slices)."""
    import torch

    import synth
    kc_dtype = "bf16" if kc_scale is None else "e4m3fn"
    out = (torch.empty((spec.B, spec.S, spec.k), dtype=torch.int32, device=dev),
           torch.empty((spec.B, spec.S, spec.k), dtype=torch.float32, device=dev))
    # the widest slice is the last one: its plan sizes the shared workspace
    pl = si.plan(spec.B, slice_rows, spec.T, spec.H, spec.D, spec.m, spec.k,
                 q_pos0=spec.S - slice_rows, kc_dtype=kc_dtype)
    ws = si.workspace(pl, dev)
    stream = torch.cuda.current_stream(dev)
    busy = 0.0
    n = 0
    for r0 in range(0, spec.S, slice_rows):
        r1 = min(spec.S, r0 + slice_rows)
        q = synth.gen_q_rows(spec, r0, r1, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        si.indexer_topk(q, kc, w[:, r0:r1], spec.m, spec.k, kc_scale=kc_scale, q_pos0=r0,
                        out=(out[0][:, r0:r1], out[1][:, r0:r1]), ws=ws)
        e1.record(stream)
        e1.synchronize()
        busy += e0.elapsed_time(e1) / 1e3
        del q
        n += 1
    torch.cuda.synchronize(dev)
    return torch.cuda.max_memory_allocated(dev), busy, n, out


def cpu_baseline(spec, x, seconds, seed=100, fp8_q=False):
    """Time the float64 oracle on sampled query rows (roughly `seconds` of work).  With
    fp8_q the oracle quantises each row's q itself, then scores the E4M3 operands."""
    import numpy as np
    import torch

    import oracle
    import synth

    try:
        import threadpoolctl
        threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()),
                      default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cpu_model = cpu_model_name()
    rows = synth.sample_rows(spec, 4096, salt=seed)
    rng = np.random.default_rng(seed)
    rng.shuffle(rows)
    kc_cpu = x["kc"].cpu()
    kc_bits = (kc_cpu.numpy() if kc_cpu.dtype == torch.uint8
               else kc_cpu.view(torch.int16).numpy().view(np.uint16))
    kc_scale = None if x["kc_scale"] is None else x["kc_scale"].cpu().numpy()
    kc_dtype = spec.kc_dtype
    done_pairs, done_rows, checked = 0, [], []
    t0 = time.perf_counter()
    while rows and time.perf_counter() - t0 < seconds:
        r = rows.pop()
        qb = x["q"][:, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        wb = x["w"][:, r:r + 1].cpu().numpy()
        t1 = time.perf_counter()
        q_dtype = "bf16"
        if fp8_q:
            qb, wb, _ = oracle.quantize_q_e4m3(qb, wb)
            q_dtype = "e4m3fn"
        idx, _ = oracle.indexer_topk(qb, kc_bits, wb, spec.m, spec.k, kc_dtype=kc_dtype,
                                     kc_scale=kc_scale, q_pos0=r, q_dtype=q_dtype)
        checked.append((r, idx[0, 0]))
        done_pairs += spec.B * oracle.visible_count(r, spec.m, spec.T)
        done_rows.append(time.perf_counter() - t1)
    elapsed = sum(done_rows)
    return {
        "value": done_pairs / elapsed if elapsed > 0 else 0.0,
        "unit": "pairs/s",
        "cores": int(threads),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"{len(done_rows)} query rows sampled uniformly over rows that see >= k keys "
                  f"(seed {seed}), float64 NumPy oracle{' (q quantised per row)' if fp8_q else ''}, "
                  f"{done_pairs} visible pairs in {elapsed:.1f} s",
    }, checked


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; 5 for long, 3 for million)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 3; 1 for long and million)")
    ap.add_argument("--workload", default="v4flash", choices=sorted(WORKLOADS))
    ap.add_argument("--key-tile", type=int, default=0)
    ap.add_argument("--query-chunk", type=int, default=0)
    ap.add_argument("--key-partition", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="bench", choices=["bench", "select-once", "copy-probe",
                                                         "summarize", "gemm-ceiling",
                                                         "kernel-table"],
                    help="select-once / copy-probe: single launches for rocprofv3 counter "
                         "runs; summarize DIR: turn rocprofv3 CSV output into the summary")
    ap.add_argument("--dir", default=None, help="rocprofv3 output root for --mode summarize")
    ap.add_argument("--timed-launches", type=int, default=5,
                    help="--mode summarize: select launches of the profiled run's timed steps")
    args = ap.parse_args(argv)
    d_steps, d_warm = DEFAULT_STEPS.get(args.workload, (10, 3))
    args.steps = d_steps if args.steps is None else args.steps
    args.warmup = d_warm if args.warmup is None else args.warmup
    if args.mode == "summarize":
        return summarize(args.dir, args.timed_launches, args.workload)
    if args.mode == "gemm-ceiling":
        return gemm_ceiling()
    if args.mode == "kernel-table":
        return kernel_table(args.dir)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(query rows would shard across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import streaming_top_selection_amd as si
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec = synth.CONFIGS[WORKLOAD_SPEC.get(args.workload, args.workload)]
    if args.workload in TWO_STAGE:
        return bench_two_stage(args, spec, dev)
    if args.workload in COMPOSE:
        return bench_compose(args, spec, dev)
    fp8_q = args.workload in FP8_Q
    capacity = None
    if args.workload == "million" and args.mode == "bench":
        # q streamed in slices, never resident whole: the peak HBM of the pages' capacity
        # run (measured first, on an empty allocator, so nothing else inflates it)
        kc0, ks0 = synth.gen_keys(spec, device=dev)
        w0 = synth.gen_w_rows(spec, device=dev)
        torch.cuda.synchronize(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        cap_peak, cap_s, cap_n, capacity_outputs = capacity_pass(si, spec, kc0, ks0, w0, dev)
        capacity = {"peak_hbm_bytes": int(cap_peak), "peak_hbm_gb": cap_peak / 1e9,
                    "indexer_seconds": cap_s, "slices": cap_n, "slice_rows": CAPACITY_SLICE_ROWS,
                    "pairs_per_s": spec.B * visible_pairs(spec.S, spec.T, spec.m) / cap_s}
        del kc0, ks0, w0
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
    x = synth.make_inputs(spec, device=dev)
    torch.cuda.synchronize(dev)
    # the peak of the timed work: inputs (already resident) + outputs + workspace; the
    # generator's temporaries are behind this reset
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    free0, total_mem = torch.cuda.mem_get_info(dev)
    input_bytes = tensor_bytes(x["q"], x["kc"], x["kc_scale"], x["w"])
    kc_dtype = spec.kc_dtype
    knobs = dict(key_tile=args.key_tile, query_chunk=args.query_chunk,
                 key_partition=args.key_partition)
    pl = si.plan(spec.B, spec.S, spec.T, spec.H, spec.D, spec.m, spec.k, 0, kc_dtype, **knobs)
    ws = si.workspace(pl, dev)
    out = (torch.empty((spec.B, spec.S, spec.k), dtype=torch.int32, device=dev),
           torch.empty((spec.B, spec.S, spec.k), dtype=torch.float32, device=dev))
    output_bytes = tensor_bytes(*out)
    stream = torch.cuda.current_stream(dev)
    # the scorer's operands: bf16 q and w, or (fp8 q) the quantiser's outputs, rewritten
    # by the quantise kernel at the start of every step
    if fp8_q:
        qop = (torch.empty(x["q"].shape, dtype=torch.uint8, device=dev),
               torch.empty(x["w"].shape, dtype=torch.float32, device=dev))
        output_bytes += tensor_bytes(*qop)
    else:
        qop = (x["q"], x["w"])
    quant_events = []

    def step(events=None):
        if fp8_q:
            if events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            si.quantize_q(x["q"], x["w"], out=qop)
            if events is not None:
                e1.record(stream)
                quant_events.append((e0, e1))
        for c in range(pl.n_chunks):
            if events is not None:
                events[c][0].record(stream)
            si.indexer_select_chunk(qop[0], x["kc"], qop[1], spec.m, spec.k, c, ws,
                                    kc_scale=x["kc_scale"], **knobs)
            if events is not None:
                events[c][1].record(stream)
            si.indexer_merge_chunk(spec.B, spec.S, spec.T, spec.H, spec.D, spec.m, spec.k, c,
                                   ws, out, kc_dtype=kc_dtype, **knobs)
            if events is not None:
                events[c][2].record(stream)

    if args.mode == "select-once":
        step()
        torch.cuda.synchronize(dev)
        si.indexer_select_chunk(qop[0], x["kc"], qop[1], spec.m, spec.k, 0, ws,
                                kc_scale=x["kc_scale"], **knobs)
        torch.cuda.synchronize(dev)
        print("select-once done", flush=True)
        return 0
    if args.mode == "copy-probe":
        a = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize(dev)
        b.copy_(a)
        torch.cuda.synchronize(dev)
        print(f"copy-probe done: {COPY_PROBE_BYTES} bytes read and written", flush=True)
        return 0

    # the staged step is the product call: check once against si_indexer_topk itself
    step()
    ref = si.indexer_topk(qop[0], x["kc"], qop[1], spec.m, spec.k, kc_scale=x["kc_scale"],
                          out=(torch.empty_like(out[0]), torch.empty_like(out[1])), ws=ws,
                          **knobs)
    torch.cuda.synchronize(dev)
    assert torch.equal(ref[0], out[0]) and torch.equal(ref[1], out[1])
    del ref
    # the keys the select stage leaves per list (for the merge's bytes), before the
    # warm-up so that the timed launches stay the last ones
    list_keys = list_lengths(si, spec, pl, ws, qop, x, knobs)
    if capacity is not None:
        assert torch.equal(capacity_outputs[0], out[0]) and \
            torch.equal(capacity_outputs[1], out[1]), "streamed-q run differs"
        del capacity_outputs
        capacity["equal_to_resident_run"] = True
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(pl.n_chunks)]
           for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    sel_ms = [e[0].elapsed_time(e[1]) for s in evs for e in s]
    mrg_ms = [e[1].elapsed_time(e[2]) for s in evs for e in s]
    peak_alloc = torch.cuda.max_memory_allocated(dev)
    free1, _ = torch.cuda.mem_get_info(dev)

    pairs = spec.B * visible_pairs(spec.S, spec.T, spec.m)
    flops = pairs * 2 * spec.H * spec.D
    step_s = wall / args.steps
    sel_mean_s = sum(sel_ms) / len(sel_ms) / 1e3
    mrg_mean_s = sum(mrg_ms) / len(mrg_ms) / 1e3
    # per step: all select launches together do the step's flops (one launch when the
    # whole workload is one query chunk)
    sel_step_s = sum(sel_ms) / args.steps / 1e3
    mrg_step_s = sum(mrg_ms) / args.steps / 1e3
    achieved_tflops = flops / sel_step_s / 1e12
    # merge: read every list the select stage left (its keys of 8 B, its count and its
    # 16-byte keep rule), write k (idx, score) pairs per row; the list lengths were read
    # back after one more select launch per chunk, outside the timed region
    import numpy as np
    merge_bytes = (list_keys * 8 + spec.B * spec.S * pl.n_partitions * (4 + 16)
                   + spec.B * spec.S * spec.k * 8)
    merge_gbps = merge_bytes / mrg_step_s / 1e9
    peak_tflops = FP8_DENSE_PEAK_TFLOPS if fp8_q else BF16_DENSE_PEAK_TFLOPS
    q_dtype = "e4m3fn" if fp8_q else "bf16"

    traffic = committed_traffic(args.workload) if not any(knobs.values()) else None
    rec = {
        "metric": METRIC,
        "value": pairs / step_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[(q_dtype, kc_dtype)],
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "B": spec.B, "S": spec.S, "T": spec.T, "H_I": spec.H, "D": spec.D, "m": spec.m,
            "k": spec.k, "q_dtype": q_dtype, "key_dtype": kc_dtype, "key_tile": pl.key_tile,
            "query_chunk": pl.query_chunk, "key_partition": pl.key_partition,
            "n_partitions": pl.n_partitions, "n_chunks": pl.n_chunks,
        },
        "visible_pairs": pairs,
        "mfma_frac": achieved_tflops / peak_tflops,
        "peak_hbm_bytes": int(peak_alloc),
        "peak_hbm_gib": peak_alloc / 2 ** 30,
        "hbm_bytes": {"inputs": input_bytes, "outputs": output_bytes,
                      "workspace": int(ws.numel()), "allocator_peak_timed": int(peak_alloc)},
        "device_mem_delta_bytes": int(free0 - free1),
        "roofline": {
            "kernel": ("select_kernel (fused E4M3 f8f6f4-MFMA scoring + running top-k)"
                       if fp8_q else "select_kernel (fused bf16 MFMA scoring + running top-k)"),
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": peak_tflops,
            "peak_dtype": "fp8 dense" if fp8_q else "bf16 dense",
            "unit": "TFLOP/s",
            "frac": achieved_tflops / peak_tflops,
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "mean_launch_ms": sel_mean_s * 1e3,
            "launches_per_step": pl.n_chunks,
            "flops_per_step": flops,
        },
        "merge": {
            "kernel": ("merge_select_sort_kernel (keep rule from the select histogram, "
                       "register bitonic sort)" if pl.n_partitions == 1 and spec.k <= 512
                       else "merge_sort_kernel (one list per row, register bitonic sort)"
                       if pl.n_partitions == 1
                       else "merge_kernel (LDS gather, select, bitonic sort)"),
            "bound": "hbm", "achieved": merge_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": merge_gbps / HBM_PEAK_GBPS,
            "mean_launch_ms": mrg_mean_s * 1e3, "bytes_per_step": merge_bytes,
            "list_keys_per_row": list_keys / (spec.B * spec.S),
        },
    }
    if fp8_q:
        # quantise: read bf16 q + w, write E4M3 q + w_eff (HBM-bound)
        nvec = spec.B * spec.S * spec.H
        qbytes = nvec * spec.D * 3 + nvec * 8
        qt = [a.elapsed_time(b) for a, b in quant_events] or [float("nan")]
        qmean = sum(qt) / len(qt) / 1e3
        rec["quantize"] = {"kernel": "quantize_q_kernel (per-(row, head) E4M3 q, w * scale)",
                           "bound": "hbm", "achieved": qbytes / qmean / 1e9,
                           "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": qbytes / qmean / 1e9 / HBM_PEAK_GBPS,
                           "mean_launch_ms": qmean * 1e3, "bytes_per_step": qbytes}
    if capacity is not None:
        rec["streamed_q_capacity_run"] = capacity
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        base, checked = cpu_baseline(spec, x, args.cpu_seconds, fp8_q=fp8_q)
        rec["cpu_baseline"] = base
        got = out[0][0].cpu().numpy()
        hits = [len((set(got[r].tolist()) & set(o.tolist())) - {-1}) /
                max(1, len(set(o.tolist()) - {-1})) for r, o in checked]
        rec["oracle_sample_recall"] = {"rows": len(checked),
                                       "mean": float(np.mean(hits)) if hits else None,
                                       "min": float(np.min(hits)) if hits else None}
        if fp8_q:
            # the quantisation's own effect: the same rows against the oracle of the
            # unquantised bf16 q (same keys)
            import oracle
            kc_c = x["kc"].cpu().numpy()
            ks_c = x["kc_scale"].cpu().numpy()
            rb = []
            for r, _ in checked[:64]:
                qb = x["q"][:, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
                oi, _ = oracle.indexer_topk(qb, kc_c, x["w"][:, r:r + 1].cpu().numpy(), spec.m,
                                            spec.k, kc_dtype=kc_dtype, kc_scale=ks_c, q_pos0=r)
                o = set(oi[0, 0].tolist()) - {-1}
                rb.append(len(set(got[r].tolist()) & o) / max(1, len(o)))
            rec["recall_vs_bf16_q_oracle"] = {"rows": len(rb), "mean": float(np.mean(rb)),
                                              "min": float(np.min(rb))}
    print(json.dumps(rec), flush=True)
    return 0


def _pmc_value(csv_dir, counter, kernel_substr):
    """Counter value of the last dispatch whose kernel name contains kernel_substr."""
    import csv
    best = None
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if counter == r["Counter_Name"] and kernel_substr in r["Kernel_Name"]:
                    d = int(r["Dispatch_Id"])
                    if best is None or d > best[0]:
                        best = (d, 0.0)
                    if d == best[0]:
                        best = (d, best[1] + float(r["Counter_Value"]))
    return None if best is None else best[1]


def _kernel_stats(csv_dir):
    import csv
    rows = []
    for path in glob.glob(os.path.join(csv_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def kernel_table(root):
    """The library's kernels in a rocprofv3 --kernel-trace --stats run under root: calls,
    total and mean duration (torch's own kernels left out)."""
    rows = [r for r in _kernel_stats(root) if "si::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | total ms | mean us |")
    print("|---|---|---|---|")
    for r in rows:
        name = r["Name"].replace("void ", "").split("(")[0]
        print(f"| {name} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
              f"{float(r['AverageNs']) / 1e3:.1f} |")
    return 0


def _dispatches(csv_dir, kernel_substr):
    """(dispatch id, duration ns) of every dispatch of a kernel in a kernel trace, in
    dispatch order."""
    import csv
    out = []
    for path in glob.glob(os.path.join(csv_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel_substr in r["Kernel_Name"]:
                    out.append((int(r["Dispatch_Id"]),
                                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return sorted(out)


def timed_launch_stats(durations_ns, timed):
    """Mean and median (us) of the last `timed` launches: the bench's timed steps come
    last, after the equality check and the warm-up launches."""
    import statistics
    d = [x / 1e3 for x in durations_ns[-timed:]] if timed > 0 else []
    if not d:
        return None
    return {"launches": len(d), "mean_us": statistics.fmean(d), "median_us": statistics.median(d)}


def summarize(root, timed=5, workload="v4flash"):
    """Prints the markdown summary of a profile directory with subdirectories trace/
    (kernel trace + stats of a bench run), clock/ (GRBM_GUI_ACTIVE + kernel trace of
    select-once), fetch/ and write/ (select-once counters) and copy_fetch/, copy_write/
    (copy-probe counters)."""
    import synth
    spec = synth.CONFIGS[WORKLOAD_SPEC.get(workload, workload)]
    flops = spec.B * visible_pairs(spec.S, spec.T, spec.m) * 2 * spec.H * spec.D
    stats = _kernel_stats(os.path.join(root, "trace"))
    sel = _pmc_value(os.path.join(root, "fetch"), "FETCH_SIZE", "select_kernel")
    wr = _pmc_value(os.path.join(root, "write"), "WRITE_SIZE", "select_kernel")
    cf = _pmc_value(os.path.join(root, "copy_fetch"), "FETCH_SIZE", "")
    cw = _pmc_value(os.path.join(root, "copy_write"), "WRITE_SIZE", "")
    fetch_scale = COPY_PROBE_BYTES / (cf * 1024) if cf else None
    write_scale = COPY_PROBE_BYTES / (cw * 1024) if cw else None
    fetch_b = sel * 1024 * fetch_scale if sel and fetch_scale else None
    write_b = wr * 1024 * write_scale if wr and write_scale else None
    print("| kernel | calls | total ms | average us | percent |")
    print("|---|---|---|---|---|")
    for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        print(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['TotalDurationNs'])/1e6:.3f} | "
              f"{float(r['AverageNs'])/1e3:.1f} | {float(r['Percentage']):.2f} |")
    print()
    disp = _dispatches(os.path.join(root, "trace"), "select_kernel")
    ts = timed_launch_stats([d for _, d in disp], timed)
    if ts:
        print(f"select_kernel, all {len(disp)} launches (us): "
              f"{', '.join(f'{d / 1e3:.1f}' for _, d in disp)}")
        print(f"select_kernel over the {ts['launches']} timed launches (the last ones): "
              f"mean {ts['mean_us']:.1f} us, median {ts['median_us']:.1f} us")
        peak = FP8_DENSE_PEAK_TFLOPS if workload in FP8_Q else BF16_DENSE_PEAK_TFLOPS
        frac = flops / (ts["mean_us"] * 1e-6) / (peak * 1e12)
        print(f"roofline: {flops:.4e} algorithmic flop per launch / {ts['mean_us']:.1f} us = "
              f"{flops / (ts['mean_us'] * 1e-6) / 1e12:.1f} TFLOP/s = {frac:.3f} of the "
              f"{peak:.0f} TFLOP/s {'fp8' if workload in FP8_Q else 'bf16'} dense peak")
    gg = _pmc_value(os.path.join(root, "clock"), "GRBM_GUI_ACTIVE", "select_kernel")
    cd = _dispatches(os.path.join(root, "clock"), "select_kernel")
    if gg and cd:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs
        ghz = gg / 8 / cd[-1][1]
        print(f"clock under the select kernel (GRBM_GUI_ACTIVE / 8 XCDs / duration of the "
              f"same dispatch, {cd[-1][1] / 1e3:.1f} us): {ghz:.2f} GHz")
    print()
    print(f"select_kernel FETCH_SIZE {sel} KiB, WRITE_SIZE {wr} KiB per launch")
    print(f"copy probe ({COPY_PROBE_BYTES} B read + written): FETCH_SIZE {cf} KiB, "
          f"WRITE_SIZE {cw} KiB -> scale fetch x{fetch_scale}, write x{write_scale}")
    mf = _pmc_value(os.path.join(root, "fetch"), "FETCH_SIZE", "merge")
    mw = _pmc_value(os.path.join(root, "write"), "WRITE_SIZE", "merge")
    if mf is not None and mw is not None and fetch_scale and write_scale:
        print(f"merge FETCH_SIZE {mf} KiB, WRITE_SIZE {mw} KiB per launch -> "
              f"{mf * 1024 * fetch_scale:.0f} B read, {mw * 1024 * write_scale:.0f} B written")
    if fetch_b is not None and write_b is not None:
        rec = {"kernel_source_sha256_16": kernel_source_hash(),
               "fetch_bytes": fetch_b, "write_bytes": write_b,
               "bytes_per_launch": fetch_b + write_b}
        print(f"<!-- traffic {json.dumps(rec)} -->")
    return 0


if __name__ == "__main__":
    sys.exit(main())
