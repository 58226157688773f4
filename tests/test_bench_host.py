"""Host-side logic of bench.py (no GPU): the one-GPU contract and the profile summarizer
that turns rocprofv3 CSVs into the per-call traffic and durations the roofline reports."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

TOPK = "void ix::(anonymous namespace)::ix_topk_partial_kernel<4, 16, 128, true>(ix::(anonymous namespace)::IxArgs)"
MERGE = "ix::(anonymous namespace)::ix_topk_merge_kernel(ix::(anonymous namespace)::IxArgs)"
ATT1 = "void ix::(anonymous namespace)::sparse_attn_kernel<128, false>(ix::(anonymous namespace)::AttnArgs)"
ATTN = "void ix::(anonymous namespace)::sparse_attn_light_kernel<128, true>(ix::(anonymous namespace)::AttnArgs)"
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, kib) in enumerate(rows):
            # two TCC instances per dispatch: the summarizer adds them
            w.writerow([i, name, counter, kib / 2])
            w.writerow([i, name, counter, kib / 2])


def test_summarizer_per_call_traffic_and_durations(tmp_path, monkeypatch):
    prof = tmp_path / "prof"
    prof.mkdir()
    # FETCH: the 1 GiB copy reads as 512 MiB (scale 2); WRITE reads as 1 GiB (scale 1)
    fetch = [(COPY, 524288.0), (TOPK, 1000.0), (TOPK, 10.0), (MERGE, 50.0), (TOPK, 1000.0),
             (TOPK, 10.0), (MERGE, 50.0), (ATT1, 300.0), (ATT1, 300.0), (ATTN, 999.0)]
    write = [(COPY, 1048576.0), (TOPK, 100.0), (TOPK, 0.0), (MERGE, 8.0), (TOPK, 100.0),
             (TOPK, 0.0), (MERGE, 8.0), (ATT1, 64.0), (ATT1, 64.0), (ATTN, 256.0)]
    _counters(prof / "fetch.csv", "FETCH_SIZE", fetch)
    _counters(prof / "write.csv", "WRITE_SIZE", write)
    with open(prof / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([TOPK, 4, 500500, 1000, 1000000, 80.0])
    with open(prof / "kt_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for name, ns in ((TOPK, 1_000_000), (MERGE, 20_000), (TOPK, 4_000), (MERGE, 5_000),
                         (TOPK, 1_000_000), (MERGE, 20_000), (TOPK, 4_000), (MERGE, 5_000),
                         (ATT1, 300_000), (ATT1, 310_000), (ATTN, 900_000)):
            w.writerow([name, t, t + ns])
            t += ns + 1000
    with open(prof / "kt.json", "w") as f:
        f.write(json.dumps({"detail": {"ix_topk_ms": 1.03, "sparse_attn_ms_per_layer": 0.31}}) + "\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    args = SimpleNamespace(summarize_profiles=(str(prof / "kt_kernel_stats.csv"), str(prof / "fetch.csv"),
                                               str(prof / "write.csv")),
                           profile_commands=("kt cmd", "fetch cmd", "write cmd"),
                           profile_bench_json=str(prof / "kt.json"))
    bench.summarize_profiles(args, "wl")
    tr = json.load(open(tmp_path / "profiles" / "traffic_wl.json"))
    # ix_topk per call: (2 sweeps + 2 recompute passes + 2 merges) / 2 sweeps
    want_topk = (2120.0 * 1024 * 2.0 + 216.0 * 1024 * 1.0) / 2
    assert tr["indexer_bytes"] == round(want_topk)
    # attention: the single-layer launches only (not the launch of several layers)
    assert tr["attention_bytes"] == round(300.0 * 1024 * 2.0 + 64.0 * 1024)
    assert tr["fetch_scale"] == 2.0 and tr["write_scale"] == 1.0
    kt = open(tmp_path / "profiles" / "kernel_trace_wl.md").read()
    # per call: (2 x 1000 + 2 x 20 + 2 x 4 + 2 x 5) us / 2 sweeps = 1029 us; attention 305 us
    assert "| `ix_topk` (sweeps, merges and recompute pass) | 2 | 1029.0 |" in kt
    assert "| `sparse_attn_kernel<128, false>(AttnArgs)` (one layer) | 2 | 305.0 |" in kt
    assert "| `sparse_attn_light_kernel` (a launch of several layers) | 1 | 900.0 |" in kt
    assert "`ix_topk` 1030.0 us" in kt
