"""Host logic of bench.py, on the CPU: the visible-pair count, the gate that keeps
counter traffic tied to the kernel sources it was measured on, the rocprofv3 summary
arithmetic, and the single-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _brute_pairs(S, T, m, q_pos0=0):
    return sum(min(T, (q_pos0 + t + 1) // m) for t in range(S))


@pytest.mark.parametrize("S,T,m,q_pos0", [(64, 16, 4, 0), (100, 30, 3, 7), (37, 5, 1, 0),
                                          (8, 0, 4, 0), (50, 1000, 2, 11)])
def test_visible_pairs_brute_force(S, T, m, q_pos0):
    assert bench.visible_pairs(S, T, m, q_pos0) == _brute_pairs(S, T, m, q_pos0)


def test_visible_pairs_closed_form():
    # S = m*T: sum_t min(T, floor((t+1)/m)) = m*T*(T-1)/2 + T, i.e. T*(2T-1) at m = 4
    for T in (1, 7, 256, 16384):
        assert bench.visible_pairs(4 * T, T, 4) == T * (2 * T - 1)


def test_traffic_gate(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "fetch_bytes": 3.0,
           "write_bytes": 4.0, "bytes_per_launch": 7.0}
    good = tmp_path / "good.md"
    good.write_text(f"text\n<!-- traffic {json.dumps(rec)} -->\n")
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", {"v4flash": str(good)})
    assert bench.committed_traffic() == rec
    stale = tmp_path / "stale.md"
    stale.write_text("<!-- traffic " + json.dumps(dict(rec, kernel_source_sha256_16="0" * 16))
                     + " -->\n")
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", {"v4flash": str(stale)})
    assert bench.committed_traffic() is None
    monkeypatch.setattr(bench, "PROFILE_SUMMARY", {"v4flash": str(tmp_path / "missing.md")})
    assert bench.committed_traffic() is None


def _write_counters(path, rows):
    path.mkdir(parents=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_scales_by_the_copy_probe(tmp_path, capsys):
    (tmp_path / "trace").mkdir()
    with open(tmp_path / "trace" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage"])
        w.writeheader()
        w.writerow(dict(Name="si::select_kernel<4, 4, 1, 2048, false>", Calls=2,
                        TotalDurationNs=2e7, AverageNs=1e7, Percentage=95.0))
    sel, mrg = "si::select_kernel<4, 4, 1, 2048, false>", "si::merge_sort_kernel<3>"
    # two select dispatches: the last one counts; counters summed over its rows
    _write_counters(tmp_path / "fetch", [
        dict(Dispatch_Id=1, Kernel_Name=sel, Counter_Name="FETCH_SIZE", Counter_Value=999),
        dict(Dispatch_Id=3, Kernel_Name=sel, Counter_Name="FETCH_SIZE", Counter_Value=600),
        dict(Dispatch_Id=3, Kernel_Name=sel, Counter_Name="FETCH_SIZE", Counter_Value=400),
        dict(Dispatch_Id=2, Kernel_Name=mrg, Counter_Name="FETCH_SIZE", Counter_Value=50)])
    _write_counters(tmp_path / "write", [
        dict(Dispatch_Id=3, Kernel_Name=sel, Counter_Name="WRITE_SIZE", Counter_Value=200),
        dict(Dispatch_Id=2, Kernel_Name=mrg, Counter_Name="WRITE_SIZE", Counter_Value=100)])
    # the copy probe reads 2^30 B and reports half of it, writes 2^30 B and reports all
    _write_counters(tmp_path / "copy_fetch", [
        dict(Dispatch_Id=1, Kernel_Name="copy", Counter_Name="FETCH_SIZE",
             Counter_Value=bench.COPY_PROBE_BYTES / 2048)])
    _write_counters(tmp_path / "copy_write", [
        dict(Dispatch_Id=1, Kernel_Name="copy", Counter_Name="WRITE_SIZE",
             Counter_Value=bench.COPY_PROBE_BYTES / 1024)])
    assert bench.summarize(str(tmp_path)) == 0
    out = capsys.readouterr().out
    assert "| si::select_kernel<4, 4, 1, 2048, false> | 2 | 20.000 | 10000.0 | 95.00 |" in out
    rec = json.loads(out.split("<!-- traffic ")[1].split(" -->")[0])
    assert rec["fetch_bytes"] == pytest.approx(1000 * 1024 * 2.0)
    assert rec["write_bytes"] == pytest.approx(200 * 1024 * 1.0)
    assert rec["bytes_per_launch"] == pytest.approx(1000 * 2048 + 200 * 1024)
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert f"-> {50 * 1024 * 2} B read, {100 * 1024} B written" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
