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
HBM_PEAK_GBPS = 8000.0              # MI355X HBM3E

WORKLOADS = {
    "v4flash": "V4-Flash indexer layer: B=1, S=65536 queries, m=4, T=16384 compressed keys, "
               "H_I=64, D=128, top-k=512, bf16 q/k with per-channel U(0.5,2) scales, "
               "fp32 w ~ N(0,1)/8, causal",
    "tiny": "Tiny indexer: B=1, S=1024, m=4, T=256, H_I=64, D=128, top-k=64",
    "small": "Small exactness check: B=2, S=8192, m=4, T=2048, H_I=64, D=128, top-k=512, 5% duplicate keys",
    "long": "Long-context: B=1, S=262144, m=4, T=65536, H_I=64, D=128, top-k=512",
}


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["si_select.hpp", "si_select_kt512_bf16.hip", "si_compact.hpp", "si_score.hpp",
                  "si_common.hpp"]
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "select_kernel_v4flash_s65536.md")
COPY_PROBE_BYTES = 1 << 30


def kernel_source_hash():
    """SHA-256 (first 16 hex digits) of the fused select kernel's sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "streaming_top_selection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per select launch from the committed counter summary, if it was taken
    on the current kernel sources (else None: the counters no longer apply)."""
    try:
        text = open(PROFILE_SUMMARY).read()
    except OSError:
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


def cpu_baseline(spec, x, seconds, seed=100):
    """Time the float64 oracle on sampled query rows (roughly `seconds` of work)."""
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
    rows = synth.sample_rows(spec, 4096, salt=seed)
    rng = np.random.default_rng(seed)
    rng.shuffle(rows)
    kc_cpu = x["kc"].cpu()
    kc_bits = (kc_cpu.numpy() if kc_cpu.dtype == torch.uint8
               else kc_cpu.view(torch.int16).numpy().view(np.uint16))
    kc_scale = None if x["kc_scale"] is None else x["kc_scale"].cpu().numpy()
    kc_dtype = "bf16" if x["kc_scale"] is None else "e4m3fn"
    done_pairs, done_rows, checked = 0, [], []
    t0 = time.perf_counter()
    while rows and time.perf_counter() - t0 < seconds:
        r = rows.pop()
        qb = x["q"][:, r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        wb = x["w"][:, r:r + 1].cpu().numpy()
        t1 = time.perf_counter()
        idx, _ = oracle.indexer_topk(qb, kc_bits, wb, spec.m, spec.k, kc_dtype=kc_dtype,
                                     kc_scale=kc_scale, q_pos0=r)
        checked.append((r, idx[0, 0]))
        done_pairs += spec.B * oracle.visible_count(r, spec.m, spec.T)
        done_rows.append(time.perf_counter() - t1)
    elapsed = sum(done_rows)
    return {
        "value": done_pairs / elapsed if elapsed > 0 else 0.0,
        "unit": "pairs/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(done_rows)} query rows sampled uniformly over rows that see >= k keys "
                  f"(seed {seed}), float64 NumPy oracle, {done_pairs} visible pairs in "
                  f"{elapsed:.1f} s",
    }, checked


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v4flash", choices=sorted(WORKLOADS))
    ap.add_argument("--key-tile", type=int, default=0)
    ap.add_argument("--query-chunk", type=int, default=0)
    ap.add_argument("--key-partition", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="bench", choices=["bench", "select-once", "copy-probe",
                                                         "summarize"],
                    help="select-once / copy-probe: single launches for rocprofv3 counter "
                         "runs; summarize DIR: turn rocprofv3 CSV output into the summary")
    ap.add_argument("--dir", default=None, help="rocprofv3 output root for --mode summarize")
    args = ap.parse_args(argv)
    if args.mode == "summarize":
        return summarize(args.dir)

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
    spec = synth.CONFIGS[args.workload]
    torch.cuda.reset_peak_memory_stats(dev)
    free0, total_mem = torch.cuda.mem_get_info(dev)
    x = synth.make_inputs(spec, device=dev)
    kc_dtype = "bf16" if x["kc_scale"] is None else "e4m3fn"
    knobs = dict(key_tile=args.key_tile, query_chunk=args.query_chunk,
                 key_partition=args.key_partition)
    pl = si.plan(spec.B, spec.S, spec.T, spec.H, spec.D, spec.m, spec.k, 0, kc_dtype, **knobs)
    ws = si.workspace(pl, dev)
    out = (torch.empty((spec.B, spec.S, spec.k), dtype=torch.int32, device=dev),
           torch.empty((spec.B, spec.S, spec.k), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for c in range(pl.n_chunks):
            if events is not None:
                events[c][0].record(stream)
            si.indexer_select_chunk(x["q"], x["kc"], x["w"], spec.m, spec.k, c, ws,
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
        si.indexer_select_chunk(x["q"], x["kc"], x["w"], spec.m, spec.k, 0, ws,
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
    ref = si.indexer_topk(x["q"], x["kc"], x["w"], spec.m, spec.k, kc_scale=x["kc_scale"], **knobs)
    torch.cuda.synchronize(dev)
    assert torch.equal(ref[0], out[0]) and torch.equal(ref[1], out[1])
    del ref

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
    # merge: read every query's kept list (min(k, n_t) keys of 8 B, one partition
    # each when n_partitions == 1) and its count, write k (idx, score) pairs per row
    import numpy as np
    t = np.arange(spec.S, dtype=np.int64)
    kept = int(np.minimum(spec.k, np.minimum(spec.T, (t + 1) // spec.m)).sum()) * spec.B
    merge_bytes = kept * 8 + spec.B * spec.S * pl.n_partitions * 4 + spec.B * spec.S * spec.k * 8
    merge_gbps = merge_bytes / mrg_step_s / 1e9

    traffic = committed_traffic() if args.workload == "v4flash" and not any(knobs.values()) \
        else None
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "B": spec.B, "S": spec.S, "T": spec.T, "H_I": spec.H, "D": spec.D, "m": spec.m,
            "k": spec.k, "key_dtype": kc_dtype, "key_tile": pl.key_tile,
            "query_chunk": pl.query_chunk, "key_partition": pl.key_partition,
            "n_partitions": pl.n_partitions, "n_chunks": pl.n_chunks,
        },
        "visible_pairs": pairs,
        "mfma_frac": achieved_tflops / BF16_DENSE_PEAK_TFLOPS,
        "peak_hbm_bytes": int(peak_alloc),
        "peak_hbm_gib": peak_alloc / 2 ** 30,
        "device_mem_delta_bytes": int(free0 - free1),
        "roofline": {
            "kernel": "select_kernel (fused bf16 MFMA scoring + running top-k)",
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": BF16_DENSE_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / BF16_DENSE_PEAK_TFLOPS,
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "mean_launch_ms": sel_mean_s * 1e3,
            "launches_per_step": pl.n_chunks,
            "flops_per_step": flops,
        },
        "merge": {
            "kernel": ("merge_sort_kernel (one list per row, register bitonic sort)"
                       if pl.n_partitions == 1 and spec.k <= 2048
                       else "merge_kernel (LDS gather, select, bitonic sort)"),
            "bound": "hbm", "achieved": merge_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": merge_gbps / HBM_PEAK_GBPS,
            "mean_launch_ms": mrg_mean_s * 1e3, "bytes_per_step": merge_bytes,
        },
    }
    if not args.no_cpu_baseline and args.cpu_seconds > 0:
        base, checked = cpu_baseline(spec, x, args.cpu_seconds)
        rec["cpu_baseline"] = base
        got = out[0][0].cpu().numpy()
        hits = [len((set(got[r].tolist()) & set(o.tolist())) - {-1}) /
                max(1, len(set(o.tolist()) - {-1})) for r, o in checked]
        rec["oracle_sample_recall"] = {"rows": len(checked),
                                       "mean": float(np.mean(hits)) if hits else None,
                                       "min": float(np.min(hits)) if hits else None}
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


def summarize(root):
    """Prints the markdown summary of a profile directory with subdirectories trace/
    (kernel trace + stats), fetch/ and write/ (select-once counters) and copy_fetch/,
    copy_write/ (copy-probe counters)."""
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
