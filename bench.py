#!/usr/bin/env python3
"""Throughput of the FP8 indexer -> top-k -> sparse-attention path on one MI355X.

A step is one IndexShare group pass over one batch of synthetic input: the selection
(FP8 MFMA indexer fused with the streaming top-k) computed once, then sparse attention
for each layer of the group over that selection (indexshare_group_fwd).  Default
workload: 128K causal prefill, batch 1, 64 indexer heads of width 128, top-2048,
16-query-head MQA of width 128, a group of 4 layers.

Prints one JSON line: query tokens/s through the whole step, the roofline of the
dominant kernel (per-kernel times measured with events on the launch stream), the
per-layer-indexing comparison (IndexShare speedup) and the CPU oracle timed on a
bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
PEAK_GRIDS = (1024, 2048, 4096)  # grids the read and gather ceilings are measured with

KERNEL_SOURCES = ["indexed_sparse_attention_ix_amd/csrc/indexer.hip",
                  "indexed_sparse_attention_ix_amd/csrc/sparse_attn.hip",
                  "indexed_sparse_attention_ix_amd/csrc/attn_common.h",
                  "indexed_sparse_attention_ix_amd/csrc/ix_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-layer", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the attention backward (detail.attention_backward)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the path only: no cache append, IndexPool, backward or measured "
                         "ceilings (the profiling runs use it so every traced launch is the path's)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings (detail.measured_peaks)")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="at most this many query rows in the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="stop the oracle's sample once this much oracle time is spent")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (reference kernel for HBM counters)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KT_STATS", "FETCH", "WRITE"),
                    help="write profiles/ summaries from rocprofv3 CSVs of this workload: "
                         "--kernel-trace --stats kernel_stats.csv, then the counter_collection.csv "
                         "of a FETCH_SIZE run and of a WRITE_SIZE run (both with "
                         "--copy-calibration); no GPU needed")
    ap.add_argument("--profile-bench-json", default=None,
                    help="the JSON line the kernel-trace run printed (quoted beside the trace)")
    ap.add_argument("--profile-commands", nargs=3, metavar=("KT_CMD", "FETCH_CMD", "WRITE_CMD"),
                    default=("", "", ""), help="the three commands, quoted into the summaries")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the decode (decode_b64_128k) and 1M-key (chunk_prefill_1m) legs")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes for the CPU baseline (at most the host's cores)")
    ap.add_argument("--cpu-baseline-child", default=None, help=argparse.SUPPRESS)
    return ap.parse_args()


COPY_BYTES = 1 << 30  # the --copy-calibration copy reads and writes this many bytes


def short_kernel_name(name):
    n = name.replace("void ", "").replace("ix::(anonymous namespace)::", "")
    n = n.replace("(ix::(anonymous namespace)::AttnArgs)", "").replace("(ix::(anonymous namespace)::IxArgs)", "")
    n = n.replace(", ix::(anonymous namespace)::AttnArgs, long)", "").replace("(ix::(anonymous namespace)::AttnArgs, long)", "")
    return n if len(n) <= 70 else n[:67] + "..."


def summarize_profiles(args, name):
    """Kernel-trace table, HBM traffic per dispatch (FETCH_SIZE / WRITE_SIZE in KiB, scaled
    by what the same counters read for a copy of known size) and profiles/traffic_<workload>.json."""
    import csv
    import collections
    kt_path, fetch_path, write_path = args.summarize_profiles
    kt_cmd, fetch_cmd, write_cmd = args.profile_commands
    stats = list(csv.DictReader(open(kt_path)))

    def per_dispatch(path, counter):
        acc = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        return [(names[d], v) for d, v in acc.items()]

    def scale(rows):
        copies = [v for n, v in rows if "copy" in n.lower()]
        if not copies:
            raise SystemExit("no copy dispatch in the counter run: use --copy-calibration")
        copy_kib = max(copies)
        return copy_kib, (COPY_BYTES / 1024.0) / copy_kib

    f_rows = per_dispatch(fetch_path, "FETCH_SIZE")
    w_rows = per_dispatch(write_path, "WRITE_SIZE")
    f_copy, f_fac = scale(f_rows)
    w_copy, w_fac = scale(w_rows)

    # Bytes per call of each path kernel.  An ix_topk call is its main sweep plus, with key
    # splits, a merge and a recompute pass whose waves mostly exit at once: its traffic is
    # the sum over all those dispatches divided by the number of main sweeps (the
    # dispatches within 10 % of the largest).  Attention: the single-layer launches (the
    # ones timed per launch; sparse_attn_light_kernel for small grids), without the small
    # combine kernel.
    def is_topk(n):
        return "ix_topk_partial_kernel" in n or "ix_topk_merge_kernel" in n

    def is_attn(n):
        return ("sparse_attn_kernel<" in n or "sparse_attn_light_kernel<" in n) and ", false>" in n

    def is_attn_group(n):  # a launch of several layers (small grids)
        return "sparse_attn_light_kernel<" in n and ", true>" in n

    def per_call(rows, fac, pick, main_key):
        sel = [(n, v) for n, v in rows if pick(n)]
        if not sel:
            return None, 0, 0.0
        mains = [v for n, v in sel if main_key in n]
        top = max(mains) if mains else 0.0
        n_main = sum(1 for v in mains if v >= 0.1 * top) or 1
        total = sum(v for _, v in sel)
        return total * 1024 * fac / n_main, n_main, total / n_main

    def traffic_bytes(pick, main_key):
        fb, n_main, f_kib = per_call(f_rows, f_fac, pick, main_key)
        wb, _, w_kib = per_call(w_rows, w_fac, pick, main_key)
        if fb is None or wb is None:
            return None, 0, 0.0, 0.0
        return round(fb + wb), n_main, f_kib, w_kib

    idx_tr = traffic_bytes(is_topk, "ix_topk_partial_kernel")
    attn_tr = traffic_bytes(is_attn, "sparse_attn")
    group_tr = traffic_bytes(is_attn_group, "sparse_attn_light_kernel")
    tr = {"workload": name, "source_hash": kernel_source_hash(),
          "indexer_bytes": idx_tr[0], "attention_bytes": attn_tr[0],
          "fetch_scale": round(f_fac, 5), "write_scale": round(w_fac, 5)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(traffic_file(name), "w") as f:
        json.dump(tr, f, indent=1)
        f.write("\n")

    # per-call durations from the per-dispatch trace next to kernel_stats.csv, by the same
    # rule as the traffic: an ix_topk call = sweeps + merges + recompute pass / main sweeps
    trace_path = kt_path.replace("kernel_stats.csv", "kernel_trace.csv")
    per_call_md = []
    if os.path.exists(trace_path):
        durs = [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                for r in csv.DictReader(open(trace_path))]
        tk = [(n, d) for n, d in durs if is_topk(n)]
        sweeps = [d for n, d in tk if "ix_topk_partial_kernel" in n]
        at = [d for n, d in durs if is_attn(n)]
        ag = [d for n, d in durs if is_attn_group(n)]
        per_call_md = ["Per call, from `kernel_trace.csv` (microseconds):", "",
                       "| call | calls | average us |", "|---|---|---|"]
        if sweeps:
            top = max(sweeps)
            n_main = sum(1 for d in sweeps if d >= 0.1 * top) or 1
            per_call_md.append(f"| `ix_topk` (sweeps, merges and recompute pass) | {n_main} | "
                               f"{sum(d for _, d in tk) / n_main:.1f} |")
        if at:
            kn = sorted({short_kernel_name(n) for n, _ in durs if is_attn(n)})
            per_call_md.append(f"| {', '.join('`%s`' % k for k in kn)} (one layer) | {len(at)} | "
                               f"{sum(at) / len(at):.1f} |")
        if ag:
            per_call_md.append(f"| `sparse_attn_light_kernel` (a launch of several layers) | {len(ag)} | "
                               f"{sum(ag) / len(ag):.1f} |")
        if args.profile_bench_json and os.path.exists(args.profile_bench_json):
            try:
                bj = json.loads(open(args.profile_bench_json).read().strip().splitlines()[-1])
                per_call_md += ["", f"`bench.py` in the same run, timed with events on the launch stream: "
                                f"`ix_topk` {bj['detail']['ix_topk_ms'] * 1e3:.1f} us, "
                                f"`sparse_attn_fwd` {bj['detail']['sparse_attn_ms_per_layer'] * 1e3:.1f} us "
                                "per layer (with the combine kernel when the selection is split)."]
            except (ValueError, KeyError, IndexError):
                pass
        per_call_md.append("")

    kt_md = [f"# Kernel trace: {name}", "",
             "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):",
             "", "```", kt_cmd, "```", ""] + per_call_md + [
             "From `kernel_stats.csv`; durations in microseconds.", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in stats[:12]:
        kt_md.append(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{name}.md"), "w") as f:
        f.write("\n".join(kt_md) + "\n")

    tm = [f"# HBM traffic per dispatch: {name}", "",
          "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the TCC instances) from two",
          "counter runs, each scaled so that the 1 GiB device copy of `--copy-calibration` reads",
          "as 1 GiB fetched and 1 GiB written.  These are L2-to-fabric bytes: reads served by the",
          "Infinity Cache count as fetched.", "",
          "```", fetch_cmd, write_cmd, "```", "",
          f"| counter | copy kernel reads (KiB) | scale |", "|---|---|---|",
          f"| FETCH_SIZE | {f_copy:.0f} | {f_fac:.4f} |",
          f"| WRITE_SIZE | {w_copy:.0f} | {w_fac:.4f} |", "",
          "Per call: `ix_topk` = its sweep plus, with key splits, the merges and the recompute",
          "pass (summed, divided by the number of sweeps); attention = one single-layer",
          "launch (`sparse_attn_kernel`, or `sparse_attn_light_kernel` for small grids; the small",
          "combine kernel of split launches excluded).", "",
          "| call | calls counted | FETCH KiB (raw) | WRITE KiB (raw) | scaled bytes per call |",
          "|---|---|---|---|---|"]
    for label, t in (("ix_topk", idx_tr), ("sparse attention (one layer)", attn_tr),
                     ("sparse_attn_light_kernel (a launch of several layers)", group_tr)):
        if t[0] is not None:
            tm.append(f"| `{label}` | {t[1]} | {t[2]:.0f} | {t[3]:.0f} | {t[0]:.4g} |")
    tm += ["", f"Kernel sources hash {tr['source_hash']} (bench.py reads these numbers only while the",
           "kernels are unchanged)."]
    with open(os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.md"), "w") as f:
        f.write("\n".join(tm) + "\n")
    print(json.dumps(tr))


def measured_peaks(dev, sh, codes=None):
    """What the chip delivers on the path's three shapes of work (ix_peaks.h): FP8 MFMA
    alone and with 4/8/12 fp32 VALU ops per MFMA (the indexer's plain epilogue is 8, its
    64-head form about 5 over 17 MFMAs per 16 useful), a 1 GiB
    device copy, and random 256-byte row gathers from a 64 MiB table (one layer's K and V
    at 128K), from a 2 GiB table (past the 256 MB Infinity Cache) and from 16 GiB (the
    footprint of the decode step's 4 layers of K and V: 64 sequences of 128K keys).

    codes: e4m3 bytes for the MFMA operands -- the workload's own indexer codes, since the
    MFMA rate depends on the operands' bit activity (power); uniform random codes if None."""
    import torch
    from indexed_sparse_attention_ix_amd import peaks as pk
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    n_ops = 34 * 64 * 32
    if codes is None:
        g = torch.Generator(device="cpu").manual_seed(77)
        r = torch.randint(0, 256, (n_ops,), generator=g, dtype=torch.int32)
        ops = torch.where((r & 0x7F) == 0x7F, torch.full_like(r, 0x38), r).to(torch.uint8).to(dev)
    else:
        flat = codes.reshape(-1)
        ops = flat.repeat((n_ops + flat.numel() - 1) // flat.numel())[:n_ops].contiguous()
    chk = torch.zeros(1, dtype=torch.float32, device=dev)
    blocks, iters = 512, 2048
    mfma = {}
    for nv in (0, 4, 8, 12):
        t = timed(lambda: pk.ix_peak_mfma_fp8(ops.data_ptr(), nv, blocks, iters, chk.data_ptr(), sh))
        mfma[str(nv)] = round(blocks * 4 * iters * 16 * 65536 / t / 1e12, 1)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: pk.ix_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh))
    copy = round(2 * nbytes / t / 1e9, 1)
    del dst
    # read-only stream of 2 GiB (past the 256 MB Infinity Cache), as the decode indexer
    # streams its keys: the best of a few grids (the rate depends on the grid by up to 20 %)
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    xr = torch.zeros(PEAK_GRIDS[-1], dtype=torch.int32, device=dev)
    read, read_grid = 0.0, None
    for blocks in PEAK_GRIDS:
        for nt in (1, 0):
            t = timed(lambda: pk.ix_peak_read(big.data_ptr(), 2 << 30, blocks, nt, xr.data_ptr(), sh))
            if (2 << 30) / t / 1e9 > read:
                read, read_grid = round((2 << 30) / t / 1e9, 1), {"blocks": blocks, "nontemporal": nt}
    # the same stream drawn by 1024 waves (256 blocks), the decode step's indexer sweep: one
    # wave per (query, key split), 64 queries x 16 splits
    read_1024 = round(max((2 << 30) / timed(lambda: pk.ix_peak_read(
        big.data_ptr(), 2 << 30, 256, nt, xr.data_ptr(), sh)) / 1e9 for nt in (1, 0)), 1)
    del src, big
    gather, gather_grid = {}, {}
    n = 1 << 25
    for label, tbytes in (("64MiB", 64 << 20), ("2GiB", 2 << 30)):
        table = torch.empty(tbytes, dtype=torch.uint8, device=dev)
        rows = torch.randint(0, tbytes // 256, (n,), generator=torch.Generator(device="cpu").manual_seed(78),
                             dtype=torch.int32)
        rows = torch.sort(rows.view(-1, 2048), dim=1).values.reshape(-1).to(dev)  # ascending per 2048, like idx rows
        gather[label] = 0.0
        for blocks in PEAK_GRIDS:
            t = timed(lambda: pk.ix_peak_gather(table.data_ptr(), tbytes, rows.data_ptr(), n, blocks,
                                                xr.data_ptr(), sh))
            if n * 256 / t / 1e9 > gather[label]:
                gather[label], gather_grid[label] = round(n * 256 / t / 1e9, 1), blocks
        del table, rows
    # 16 segments of 1 GiB, each load step of a wave in one of them (ix_peak_gather_wide)
    seg = 1 << 30
    table = torch.empty(16 * seg, dtype=torch.uint8, device=dev)
    rows = torch.randint(0, seg // 256, (n,), generator=torch.Generator(device="cpu").manual_seed(79),
                         dtype=torch.int32)
    rows = torch.sort(rows.view(-1, 2048), dim=1).values.reshape(-1).to(dev)
    # (ordinary and non-temporal loads: from HBM the hint helps, as it does the decode
    # attention's row loads)
    gather["16GiB"] = 0.0
    for blocks in PEAK_GRIDS:
        for nt in (0, 1):
            t = timed(lambda: pk.ix_peak_gather_wide(table.data_ptr(), seg, 16, rows.data_ptr(), n,
                                                     blocks, nt, xr.data_ptr(), sh))
            if n * 256 / t / 1e9 > gather["16GiB"]:
                gather["16GiB"] = round(n * 256 / t / 1e9, 1)
                gather_grid["16GiB"] = {"blocks": blocks, "nontemporal": nt}
    del table, rows
    return {"fp8_mfma_tflops_by_valu_per_mfma": mfma, "copy_GB_per_s": copy,
            "read_GB_per_s": read, "read_grid": read_grid, "read_GB_per_s_1024_waves": read_1024, "gather_256B_rows_GB_per_s": gather,
            "gather_grid": gather_grid}


def time_calls(fn, stream, reps, warmup=1, before=None):
    """ms per call of fn, timed with events on `stream`: the average over reps back-to-back
    calls; or, with before(r) given (run ahead of call r, outside the timed interval), the
    median of the calls timed one by one."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if before is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r in range(reps):
        before(r)
        ev[r][0].record(stream)
        fn()
        ev[r][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]  # the median: one-off stalls of a single call do not move it


def time_after(fn, before, stream, reps, warmup=1):
    """ms of fn run straight after before(r) on `stream`, with no event between the two: the
    median of before + fn, each pair timed with events around it, minus the median of before
    alone.  An event recorded between the two would charge fn the gap it adds (its dispatch
    then starts from an idle queue); the kernel trace's duration of fn is what this measures."""
    import torch
    for _ in range(warmup):
        before(0)
        fn()
    torch.cuda.synchronize()

    def med(call):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for r in range(reps):
            ev[r][0].record(stream)
            call(r)
            ev[r][1].record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return ts[len(ts) // 2]

    def both(r):
        before(r)
        fn()
    return med(both) - med(before)


def gather_ceiling(pk, kc, vc, idx, kv_len, wl, stream, reps, split_options, before=None):
    """(ms, splits, blocks per CU) of the fastest ix_peak_gather_selection over split_options
    and occupancy limits (none, or 2 blocks per CU as the attention runs): the K and V rows of
    this selection read exactly as the attention reads them, with nothing computed."""
    import torch
    xr = torch.zeros(wl.B * wl.T * wl.H_kv * max(split_options), dtype=torch.int32,
                     device=idx.device)
    sh = stream.cuda_stream
    best = None
    for sp in split_options:
        for occ in (0, 2):
            ms = time_calls(lambda: pk.ix_peak_gather_selection(
                kc, vc, idx.data_ptr(), kv_len, wl.B, wl.T, wl.S, wl.H_kv, wl.d, wl.k, sp, occ,
                xr.data_ptr(), sh), stream, reps, before=before)
            if best is None or ms < best[0]:
                best = (ms, sp, occ)
    return best


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and blank lines are left out, so that a
    comment edit does not invalidate counters taken with the same code."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def indexer_bytes(wl):
    """Bytes the indexer must move at least once: each sequence's visible indexer-key rows,
    the queries' indexer rows and head weights, and the index rows it writes."""
    keys = 0
    for b in range(wl.B):
        keys += max(0, min(wl.pos0_list()[b] + wl.T, wl.kv_len_list()[b]))
    return keys * wl.d_I + wl.B * wl.T * (wl.H_I * (wl.d_I + 4) + wl.k * 4)


def algorithmic_work(wl):
    """Indexer flops (2*H_I*d_I per visible pair) and attention bytes per layer
    (gathered K and V rows, plus q, out and the index rows)."""
    pairs = 0
    sel = 0
    for b in range(wl.B):
        for_t = [wl.visible(b, t) for t in range(wl.T)] if wl.T <= 8192 else None
        if for_t is None:
            # closed form for pos0 + t + 1 clipped at kv_len
            import numpy as np
            n = np.minimum(np.arange(wl.T, dtype=np.int64) + wl.pos0_list()[b] + 1,
                           wl.kv_len_list()[b]).clip(min=0)
            pairs += int(n.sum())
            sel += int(np.minimum(n, wl.k).sum())
        else:
            pairs += sum(for_t)
            sel += sum(min(wl.k, n) for n in for_t)
    flops = 2.0 * wl.H_I * wl.d_I * pairs
    gathered = sel * 2.0 * wl.d * 2 * wl.H_kv
    other = wl.B * wl.T * (2.0 * wl.H_q * wl.d * 2 + wl.k * 4)
    return flops, gathered + other, pairs, sel


def cpu_sample(wl, n_max):
    """The oracle's sample of query rows as chunks [(b, rows)], the fixed rows first: rows 0
    and T-1 of the first sequence and rows k-2, k-1, k (which see fewer than, exactly and one
    more than k keys when the chunk starts at position 0), then rows drawn uniformly (seed
    1234); a decode step (T = 1) samples whole sequences.  Chunks hold up to 4 rows of one
    sequence, so the work spreads over the workers."""
    import numpy as np
    rng = np.random.default_rng(1234)
    n_max = min(n_max, wl.B * wl.T)
    if wl.T == 1:
        return [(b, [0]) for b in range(n_max)], []
    special = sorted({t for t in (0, wl.k - 2, wl.k - 1, wl.k, wl.T - 1) if 0 <= t < wl.T})
    flat = rng.choice(wl.B * wl.T, size=n_max, replace=False)
    picks = [p for p in dict.fromkeys((int(f) // wl.T, int(f) % wl.T) for f in flat)
             if not (p[0] == 0 and p[1] in special)][:max(0, n_max - len(special))]
    chunks = [(0, special)]
    by_seq = {}
    for b, t in picks:
        by_seq.setdefault(b, []).append(t)
    rest = [(b, sorted(ts[i:i + 4])) for b, ts in sorted(by_seq.items()) for i in range(0, len(ts), 4)]
    order = rng.permutation(len(rest))
    return chunks + [rest[i] for i in order], special


def cpu_baseline(args, wl, name, ind, layers, dev):
    """The oracle timed on the host's cores.  The sampled rows' inputs (the same bytes the GPU
    read) go to a temporary folder; a child process that never touches the GPU loads them and
    runs the oracle's chunks over a pool of worker processes forked from it until
    --cpu-seconds of wall time, then on one thread alone for a quarter of that."""
    import shutil
    import subprocess
    import tempfile

    import numpy as np
    import torch

    from indexed_sparse_attention_ix_amd import synth
    n_seq_max = 8 if wl.B > 1 else 1        # caches of a few sequences only (decode: 272 MiB each)
    chunks, special = cpu_sample(wl, args.cpu_rows if wl.T > 1 else n_seq_max)
    chunks = [(b, rows) for b, rows in chunks if b < n_seq_max]
    seqs = sorted({b for b, _ in chunks})
    tmp = tempfile.mkdtemp(prefix="ix_cpu_baseline_")
    try:
        arrays = {"q_pos0": ind["q_pos0"].cpu().numpy(), "kv_len": ind["kv_len"].cpu().numpy()}
        for b in seqs:
            rows = sorted({t for bb, rs in chunks if bb == b for t in rs})
            r = torch.tensor(rows, device=dev)
            arrays[f"rows_{b}"] = np.array(rows, dtype=np.int64)
            arrays[f"k_I_{b}"] = ind["k_I"][b].cpu().numpy()
            arrays[f"q_I_{b}"] = ind["q_I"][b, r].cpu().numpy()
            arrays[f"w_{b}"] = ind["w"][b, r].cpu().numpy()
            for l, Lr in enumerate(layers):
                arrays[f"q_{b}_{l}"] = synth.bf16_bits(Lr["q"][b, r])
                arrays[f"K_{b}_{l}"] = synth.bf16_bits(Lr["K"][b])
                arrays[f"V_{b}_{l}"] = synth.bf16_bits(Lr["V"][b])
        np.savez(os.path.join(tmp, "inputs.npz"), **arrays)
        del arrays
        workers = max(1, min(args.cpu_workers, os.cpu_count() or 1))
        plan = {"chunks": chunks, "seqs": seqs, "T": wl.T, "S": wl.S, "H_I": wl.H_I, "d_I": wl.d_I,
                "H_q": wl.H_q, "H_kv": wl.H_kv, "d": wl.d, "k": wl.k, "layers": wl.layers,
                "sm_scale": wl.sm_scale, "seconds": args.cpu_seconds, "workers": workers}
        with open(os.path.join(tmp, "plan.json"), "w") as f:
            json.dump(plan, f)
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", tmp],
                             capture_output=True, text=True, timeout=30 + 4 * args.cpu_seconds + 120)
        if res.returncode != 0:
            raise RuntimeError(f"CPU baseline child failed:\n{res.stdout[-2000:]}\n{res.stderr[-2000:]}")
        out = json.loads(res.stdout.strip().splitlines()[-1])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    what = (f"the first {out['rows']} sequences' decode queries" if wl.T == 1 else
            f"{out['rows']} query rows ({len(special)} fixed: t = {special} of sequence 0; "
            f"the rest drawn uniformly, in chunks of up to 4 rows)")
    return {"value": round(out["rows"] / out["wall_s"], 3), "unit": "query tokens/s",
            "cores": out["workers"], "kind": "oracle",
            "sample": f"{what} from {name} (seed 1234): fp64 scores, selection and "
                      f"{wl.layers}-layer attention per row, {out['workers']} worker processes "
                      f"with one BLAS thread each, {out['wall_s']:.1f} s of wall time",
            "host_cpus": os.cpu_count(),
            "one_thread_value": round(out["one_rows"] / out["one_s"], 3) if out["one_s"] else None,
            "one_thread_sample": f"the first {out['one_rows']} of the same rows on one thread, "
                                 f"{out['one_s']:.1f} s"}


_CHILD = {}


def _child_chunk(ci):
    """One chunk of the oracle in a worker (inputs inherited from the child process)."""
    import numpy as np
    from oracle import ix_oracle as O
    P, D = _CHILD["plan"], _CHILD["data"]
    if time.time() > _CHILD["deadline"]:
        return 0, 0.0, 0.0
    b, rows = P["chunks"][ci]
    pos = {t: i for i, t in enumerate(D[f"rows_{b}"].tolist())}
    sel = [pos[t] for t in rows]
    T = P["T"]
    qI = np.zeros((1, T, P["H_I"], P["d_I"]), dtype=np.uint8)   # only the chunk's rows are set
    w = np.zeros((1, T, P["H_I"]), dtype=np.float32)
    qI[0, rows] = D[f"q_I_{b}"][sel]
    w[0, rows] = D[f"w_{b}"][sel]
    indexer = {"q_I": qI, "k_I": D[f"k_I_{b}"][None], "w": w,
               "q_pos0": D["q_pos0"][b:b + 1], "kv_len": D["kv_len"][b:b + 1]}
    layers = []
    for l in range(P["layers"]):
        q = np.zeros((1, T, P["H_q"], P["d"]), dtype=np.uint16)
        q[0, rows] = D[f"q_{b}_{l}"][sel]
        layers.append({"q": q, "K": D[f"K_{b}_{l}"][None], "V": D[f"V_{b}_{l}"][None]})
    t0 = time.time()
    O.indexshare_group(indexer, layers, P["k"], 0, rows, P["sm_scale"])
    return len(rows), t0, time.time()


def _child_init():
    from threadpoolctl import threadpool_limits
    _CHILD["limits"] = threadpool_limits(limits=1)


def cpu_baseline_child(path):
    """Entry of the CPU-baseline child process: no GPU is touched here or in its workers."""
    import multiprocessing as mp

    import numpy as np
    plan = json.load(open(os.path.join(path, "plan.json")))
    with np.load(os.path.join(path, "inputs.npz")) as z:
        data = {k: z[k] for k in z.files}
    _CHILD.update(plan=plan, data=data)
    start = time.time()
    _CHILD["deadline"] = start + plan["seconds"]
    with mp.get_context("fork").Pool(plan["workers"], initializer=_child_init) as pool:
        res = list(pool.imap(_child_chunk, range(len(plan["chunks"]))))
    done = [r for r in res if r[0] > 0]
    rows = sum(r[0] for r in done)
    wall = max(r[2] for r in done) - start
    # the same chunks on one thread, for a quarter of the time
    from threadpoolctl import threadpool_limits
    one_rows, one_s = 0, 0.0
    _CHILD["deadline"] = float("inf")
    with threadpool_limits(limits=1):
        for ci in range(len(plan["chunks"])):
            n, t0, t1 = _child_chunk(ci)
            one_rows, one_s = one_rows + n, one_s + (t1 - t0)
            if one_s >= max(2.0, plan["seconds"] / 4):
                break
    print(json.dumps({"rows": rows, "wall_s": wall, "workers": plan["workers"],
                      "one_rows": one_rows, "one_s": one_s}), flush=True)


def run_leg(name, dev, steps):
    """The benchmark spec's other two figures, each on its own workload, after the main one: the
    decode step (64 sequences against 128K-token caches), whose attention gathers really go
    to HBM (4 GiB of K and V per layer), timed with the caches flushed; and the 1M-key
    chunked prefill, where IndexShare's one indexer per group of 4 layers is compared with
    indexing every layer.  Returns a dict of timings and rates (inputs resident in HBM)."""
    import torch

    from indexed_sparse_attention_ix_amd import binding as bd
    from indexed_sparse_attention_ix_amd import peaks as pk
    from indexed_sparse_attention_ix_amd import synth
    from indexed_sparse_attention_ix_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    L = wl.layers
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ind = synth.indexer_inputs(wl, device=dev)
    layers = [synth.attention_inputs(wl, layer=l, device=dev) for l in range(L)]
    a = bd.indexer_args(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx = torch.empty((wl.B, wl.T, wl.k), dtype=torch.int32, device=dev)
    outs = [torch.empty_like(Lr["q"]) for Lr in layers]
    ws_bytes = bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    qp = [Lr["q"].data_ptr() for Lr in layers]
    kp = [Lr["K"].data_ptr() for Lr in layers]
    vp = [Lr["V"].data_ptr() for Lr in layers]
    op = [o.data_ptr() for o in outs]
    kvl = ind["kv_len"].data_ptr()
    topk_ws = bd.ix_topk_workspace_bytes(a, wl.k)
    attn_ws = bd.sparse_attn_workspace_bytes(wl.B, wl.T, wl.H_q, wl.H_kv, wl.d, wl.k)
    reps = max(steps, 20 if wl.T > 1 else 50)

    def group_step():
        bd.indexshare_group_fwd(a, wl.k, L, qp, kp, vp, op, None, wl.H_q, wl.H_kv, wl.d,
                                wl.sm_scale, idx.data_ptr(), ws.data_ptr(), ws_bytes, sh)

    def attn(l):
        bd.sparse_attn_fwd(qp[l], kp[l], vp[l], idx.data_ptr(), kvl, wl.B, wl.T, wl.S, wl.H_q,
                           wl.H_kv, wl.d, wl.k, wl.sm_scale, op[l], 0,
                           ws.data_ptr() if attn_ws else 0, attn_ws, sh)

    ms_group = time_calls(group_step, stream, reps, warmup=3)
    ms_topk = time_calls(lambda: bd.ix_topk(a, wl.k, idx.data_ptr(), 0, ws.data_ptr(), topk_ws, sh),
                         stream, reps)
    ms_attn = time_calls(lambda: attn(0), stream, reps)
    flops, attn_bytes, pairs, sel = algorithmic_work(wl)
    ib = indexer_bytes(wl)
    # the layers' attention over the shared selection in one call, as the group step runs it
    gws = bd.sparse_attn_group_workspace_bytes(wl.B, wl.T, wl.H_q, wl.H_kv, wl.d, wl.k, L)

    def attn_group():
        bd.sparse_attn_group_fwd(L, qp, kp, vp, op, None, idx.data_ptr(), kvl, wl.B, wl.T, wl.S,
                                 wl.H_q, wl.H_kv, wl.d, wl.k, wl.sm_scale,
                                 ws.data_ptr() if gws else 0, gws, sh)
    ms_attn_group = time_calls(attn_group, stream, reps)
    # cold: a 512 MiB buffer (twice the Infinity Cache) read before every call, as a decode
    # step's selection streams its keys before the attention (a written buffer would leave
    # the caches full of dirty lines whose write-backs no step pays)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    xr = torch.zeros(4096, dtype=torch.int32, device=dev)
    n_cold = 10

    def flush(r):
        pk.ix_peak_read(scratch.data_ptr(), 512 << 20, 1024, 0, xr.data_ptr(), sh)
    ms_attn_cold = time_calls(lambda: attn(0), stream, n_cold, before=flush)
    ms_attn_group_cold = time_calls(attn_group, stream, n_cold, before=flush)
    # the same calls issued straight after the flush (no event between): the kernels' own time
    ms_attn_cold_b2b = time_after(lambda: attn(0), flush, stream, n_cold)
    ms_attn_group_cold_b2b = time_after(attn_group, flush, stream, n_cold)
    ms_group_cold = time_calls(group_step, stream, n_cold, before=flush)
    ms_topk_cold = time_calls(lambda: bd.ix_topk(a, wl.k, idx.data_ptr(), 0, ws.data_ptr(), topk_ws,
                                                 sh), stream, n_cold, before=flush)
    split_opts = [1] if wl.B * wl.T * wl.H_kv >= 1024 else [1, 2, 4, 8, 16]
    c_ms, c_sp, c_occ = gather_ceiling(pk, kp[0], vp[0], idx, kvl, wl, stream, n_cold, split_opts,
                                       before=flush)
    del scratch, xr
    # per-layer indexing: every layer with its own indexer inputs and its own top-k
    inds = [ind] + [synth.indexer_inputs(wl, layer=l, device=dev) for l in range(1, L)]
    aa = [bd.indexer_args(x["q_I"], x["k_I"], x["w"], x["q_pos0"], x["kv_len"]) for x in inds]

    def per_layer_step():
        for l in range(L):
            bd.ix_topk(aa[l], wl.k, idx.data_ptr(), 0, ws.data_ptr(), topk_ws, sh)
            attn(l)
    ms_pl = time_calls(per_layer_step, stream, max(2, reps // 2))
    gbs_cold = attn_bytes / (ms_attn_cold / 1e3) / 1e9
    gbs_group_cold = L * attn_bytes / (ms_attn_group_cold / 1e3) / 1e9
    gbs_cold_b2b = attn_bytes / (ms_attn_cold_b2b / 1e3) / 1e9
    gbs_group_cold_b2b = L * attn_bytes / (ms_attn_group_cold_b2b / 1e3) / 1e9
    out = {"workload": name, "B": wl.B, "T": wl.T, "S": wl.S, "k": wl.k, "layers": L,
           "group_ms": round(ms_group, 4), "group_ms_cold": round(ms_group_cold, 4),
           "query_tokens_per_s": round(wl.B * wl.T / (ms_group / 1e3), 1),
           "per_layer_indexing_ms": round(ms_pl, 4), "indexshare_speedup": round(ms_pl / ms_group, 3),
           "ix_topk_ms": round(ms_topk, 4), "ix_topk_ms_cold": round(ms_topk_cold, 4),
           "indexer_tflop": round(flops / 1e12, 3),
           # QK^T and PV over the kept pairs, every query head: 4 flop per (pair, head, d)
           "attention_tflop_per_layer": round(sel * wl.H_q * wl.d * 4 / 1e12, 4),
           "indexer_fp8_frac": round(flops / (ms_topk / 1e3) / 1e12 / PEAK_FP8_TFLOPS, 4),
           "indexer_bytes": ib,
           "indexer_hbm_frac_cold": round(ib / (ms_topk_cold / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
           "attention_ms_per_layer": round(ms_attn, 4),
           "attention_ms_per_layer_cold": round(ms_attn_cold, 4),
           "attention_gb_per_layer": round(attn_bytes / 1e9, 4),
           "attention_GB_per_s_cold": round(gbs_cold, 1),
           "attention_hbm_frac_cold": round(gbs_cold / PEAK_HBM_GBS, 4),
           "group_attention_ms": round(ms_attn_group, 4),
           "group_attention_ms_cold": round(ms_attn_group_cold, 4),
           "group_attention_ms_per_layer_cold": round(ms_attn_group_cold / L, 4),
           "group_attention_GB_per_s_cold": round(gbs_group_cold, 1),
           "group_attention_hbm_frac_cold": round(gbs_group_cold / PEAK_HBM_GBS, 4),
           "attention_ms_per_layer_cold_back_to_back": round(ms_attn_cold_b2b, 4),
           "attention_hbm_frac_cold_back_to_back": round(gbs_cold_b2b / PEAK_HBM_GBS, 4),
           "group_attention_ms_per_layer_cold_back_to_back": round(ms_attn_group_cold_b2b / L, 4),
           "group_attention_GB_per_s_cold_back_to_back": round(gbs_group_cold_b2b, 1),
           "group_attention_hbm_frac_cold_back_to_back": round(gbs_group_cold_b2b / PEAK_HBM_GBS, 4),
           "gather_ceiling_cold": {"ms": round(c_ms, 4), "splits": c_sp,
                                   "blocks_per_cu": c_occ or None,
                                   "GB_per_s": round(attn_bytes / (c_ms / 1e3) / 1e9, 1),
                                   "attention_frac": round(c_ms / ms_attn_cold, 4)},
           "flush": "512 MiB buffer read before each cold call, outside the events; "
                    "back_to_back: the call issued straight after the flush, flush time "
                    "subtracted"}
    del inds, aa, ind, layers, outs, ws, idx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: the path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_baseline_child)
        return
    from indexed_sparse_attention_ix_amd.workloads import BENCH_WORKLOAD, WORKLOADS
    if args.summarize_profiles:
        summarize_profiles(args, args.workload or BENCH_WORKLOAD)
        return

    import numpy as np
    import torch

    from indexed_sparse_attention_ix_amd import binding as bd
    from indexed_sparse_attention_ix_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bd.load()  # fails loudly if libix.so is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    name = args.workload or BENCH_WORKLOAD
    wl = WORKLOADS[name]
    L = wl.layers

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    # ---------------------------------------------------------------- inputs in HBM
    ind = synth.indexer_inputs(wl, device=dev)
    layers = [synth.attention_inputs(wl, layer=l, device=dev) for l in range(L)]
    a = bd.indexer_args(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx = torch.empty((wl.B, wl.T, wl.k), dtype=torch.int32, device=dev)
    outs = [torch.empty_like(Lr["q"]) for Lr in layers]
    ws_bytes = bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    qp = [Lr["q"].data_ptr() for Lr in layers]
    kp = [Lr["K"].data_ptr() for Lr in layers]
    vp = [Lr["V"].data_ptr() for Lr in layers]
    op = [o.data_ptr() for o in outs]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def group_step():
        bd.indexshare_group_fwd(a, wl.k, L, qp, kp, vp, op, None, wl.H_q, wl.H_kv, wl.d,
                                wl.sm_scale, idx.data_ptr(), ws.data_ptr(), ws_bytes, sh)

    # ---------------------------------------------------------------- timed region
    for _ in range(args.warmup):
        group_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        group_step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    tokens = wl.B * wl.T
    value = tokens / (ms / 1e3)

    # ---------------------------------------------------------------- per-kernel times
    # the same launches as the group entry point, bracketed by events on its stream
    topk_ws = bd.ix_topk_workspace_bytes(a, wl.k)
    attn_ws = bd.sparse_attn_workspace_bytes(wl.B, wl.T, wl.H_q, wl.H_kv, wl.d, wl.k)
    reps = max(2, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 2)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        bd.ix_topk(a, wl.k, idx.data_ptr(), 0, ws.data_ptr(), topk_ws, sh)
        ev[r][1].record(stream)
        for l in range(L):
            bd.sparse_attn_fwd(qp[l], kp[l], vp[l], idx.data_ptr(), ind["kv_len"].data_ptr(),
                               wl.B, wl.T, wl.S, wl.H_q, wl.H_kv, wl.d, wl.k, wl.sm_scale,
                               op[l], 0, ws.data_ptr() if attn_ws else 0, attn_ws, sh)
            ev[r][2 + l].record(stream)
    torch.cuda.synchronize()
    topk_times = [ev[r][0].elapsed_time(ev[r][1]) for r in range(reps)]
    attn_times = [ev[r][1 + l].elapsed_time(ev[r][2 + l]) for r in range(reps) for l in range(L)]
    t_topk = sum(topk_times) / reps
    t_attn = sum(attn_times) / (reps * L)

    flops, attn_bytes, pairs, sel = algorithmic_work(wl)
    idx_tflops = flops / (t_topk / 1e3) / 1e12
    attn_gbs = attn_bytes / (t_attn / 1e3) / 1e9
    ib = indexer_bytes(wl)
    if flops / ib >= PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):  # above the FP8 ridge
        idx_roof = {"bound": "mfma", "achieved": round(idx_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(idx_tflops / PEAK_FP8_TFLOPS, 4)}
    else:  # decode-like: the key rows are read once for few queries
        gbs = ib / (t_topk / 1e3) / 1e9
        idx_roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "fp8_tflops": round(idx_tflops, 2)}
    attn_roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(attn_gbs / PEAK_HBM_GBS, 4)}
    traffic = {"indexer": None, "attention": None}
    if os.path.exists(traffic_file(name)):
        try:
            tr = json.load(open(traffic_file(name)))
            if tr.get("source_hash") == kernel_source_hash() and tr.get("workload") == name:
                traffic = {"indexer": tr.get("indexer_bytes"), "attention": tr.get("attention_bytes")}
        except (OSError, ValueError):
            pass
    idx_roof["traffic"] = traffic["indexer"]
    attn_roof["traffic"] = traffic["attention"]
    # the counter-measured bytes as a rate and an HBM fraction too (for the gathers, part of
    # them come from the Infinity Cache, which the counters count as fabric traffic)
    for roof, tb, tm in ((idx_roof, traffic["indexer"], t_topk), (attn_roof, traffic["attention"], t_attn)):
        if tb:
            roof["traffic_GB_per_s"] = round(tb / (tm / 1e3) / 1e9, 1)
            roof["traffic_frac"] = round(tb / (tm / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
    # The attention's own ceiling: ix_peak_gather_selection reads exactly the rows of this
    # selection with the attention's block shape and order and computes nothing, under the
    # same conditions (back-to-back launches).  Where a layer's K and V fit in the Infinity
    # Cache (prefill up to 128K) the gathers are served from the caches, faster than HBM
    # could: the bound is then "cache", against that measured ceiling, not the HBM peak.
    from indexed_sparse_attention_ix_amd import peaks as pk
    split_opts = [1] if wl.B * wl.T * wl.H_kv >= 1024 else [1, 2, 4, 8, 16]
    t_ceil, sp_ceil, occ_ceil = gather_ceiling(pk, kp[0], vp[0], idx, ind["kv_len"].data_ptr(), wl,
                                               stream, reps, split_opts)
    ceil_gbs = attn_bytes / (t_ceil / 1e3) / 1e9
    attn_roof["gather_ceiling"] = {"ms": round(t_ceil, 4), "GB_per_s": round(ceil_gbs, 1),
                                   "splits": sp_ceil, "blocks_per_cu": occ_ceil or None,
                                   "frac": round(t_ceil / t_attn, 4)}
    if attn_gbs > PEAK_HBM_GBS:
        attn_roof.update(bound="cache", peak=round(ceil_gbs, 1), frac=round(t_ceil / t_attn, 4),
                         peak_source="measured: ix_peak_gather_selection, the same rows gathered "
                                     "with nothing computed",
                         hbm_frac_if_all_from_hbm=round(attn_gbs / PEAK_HBM_GBS, 4))
    dominant_is_indexer = t_topk >= t_attn * L
    roofline = idx_roof if dominant_is_indexer else attn_roof
    roofline = dict(roofline, kernel="ix_topk (indexer + selection)" if dominant_is_indexer
                    else "sparse_attn_fwd")

    # ---------------------------------------------------------------- cold attention
    # Where one layer's K and V exceed the 256 MB Infinity Cache (decode, the 1M chunk) the
    # gathers are HBM-bound: time the attention also after reading a 512 MiB buffer before
    # every launch, so no row is left in the caches from the previous launch.
    attn_cold = None
    kv_layer_bytes = 2 * wl.B * wl.S * wl.H_kv * wl.d * 2
    if not args.no_extras and kv_layer_bytes > (256 << 20):
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        xr = torch.zeros(4096, dtype=torch.int32, device=dev)
        n_cold = max(3, min(reps, 10))
        evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_cold)]
        for r in range(n_cold):
            pk.ix_peak_read(scratch.data_ptr(), 512 << 20, 1024, 0, xr.data_ptr(), sh)
            evc[r][0].record(stream)
            bd.sparse_attn_fwd(qp[0], kp[0], vp[0], idx.data_ptr(), ind["kv_len"].data_ptr(),
                               wl.B, wl.T, wl.S, wl.H_q, wl.H_kv, wl.d, wl.k, wl.sm_scale,
                               op[0], 0, ws.data_ptr() if attn_ws else 0, attn_ws, sh)
            evc[r][1].record(stream)
        torch.cuda.synchronize()
        t_cold = sum(a_.elapsed_time(b_) for a_, b_ in evc) / n_cold
        attn_cold = {"ms_per_layer": round(t_cold, 4),
                     "GB_per_s": round(attn_bytes / (t_cold / 1e3) / 1e9, 1),
                     "frac_of_hbm_peak": round(attn_bytes / (t_cold / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                     "flush": "512 MiB buffer read before each launch"}
        del scratch, xr

    # ---------------------------------------------------------------- cache append (producer)
    # The step before the indexer in a serving loop: this step's T tokens per sequence go
    # into the group's FP8 key cache (rounded from fp32) and every layer's K/V caches.  The
    # new rows are the ones already at those positions, so the caches stay byte-identical.
    append = None
    p0s = wl.pos0_list()
    if (not args.no_extras and all(p == p0s[0] for p in p0s) and p0s[0] >= 0
            and p0s[0] + wl.T <= wl.S):
        p0 = p0s[0]
        pos_t = torch.full((wl.B,), p0, dtype=torch.int32, device=dev)
        kn = ind["k_I"][:, p0:p0 + wl.T].view(torch.float8_e4m3fn).float().contiguous()
        kvn = [(Lr["K"][:, p0:p0 + wl.T].contiguous(), Lr["V"][:, p0:p0 + wl.T].contiguous())
               for Lr in layers]

        def append_step():
            for l in range(L):
                Kn, Vn = kvn[l]
                bd.ix_append_kv(kn.data_ptr() if l == 0 else 0, Kn.data_ptr(), Vn.data_ptr(),
                                pos_t.data_ptr(), wl.B, wl.T, wl.S, wl.d_I, wl.H_kv, wl.d,
                                ind["k_I"].data_ptr() if l == 0 else 0, layers[l]["K"].data_ptr(),
                                layers[l]["V"].data_ptr(), sh)
        append_step()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            append_step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_app = e0.elapsed_time(e1) / reps
        rows = wl.B * wl.T
        moved = rows * (wl.d_I * 5 + L * 2 * 2 * wl.H_kv * wl.d * 2)  # read + write
        append = {"ms": round(ms_app, 4), "GB_per_s": round(moved / (ms_app / 1e3) / 1e9, 1),
                  "tokens": rows, "launches": 2 + (L - 1)}
        del kn, kvn

    # ---------------------------------------------------------------- IndexPool
    # The same selection budget over block keys (4 consecutive indexer keys pooled into
    # one): pooling pre-pass + block top-k of k/4 blocks expanded to k token positions.
    indexpool = None
    if not args.no_extras and wl.k % 4 == 0:
        pool, kb = 4, wl.k // 4
        kpool = torch.empty((wl.B, (wl.S + pool - 1) // pool, wl.d_I), dtype=torch.uint8, device=dev)
        ap = bd.IndexerArgs(ind["q_I"].data_ptr(), kpool.data_ptr(), ind["w"].data_ptr(),
                            ind["q_pos0"].data_ptr(), ind["kv_len"].data_ptr(), wl.B, wl.T, wl.S,
                            wl.H_I, wl.d_I)
        pw = bd.ix_topk_pooled_workspace_bytes(ap, pool, kb)
        pws = torch.empty(max(pw, 256), dtype=torch.uint8, device=dev)
        idx_p = torch.empty_like(idx)

        def pool_pass():
            bd.ix_pool_keys(ind["k_I"].data_ptr(), ind["kv_len"].data_ptr(), wl.B, wl.S, wl.d_I,
                            pool, kpool.data_ptr(), sh)

        def pooled_topk():
            bd.ix_topk_pooled(ap, pool, kb, idx_p.data_ptr(), pws.data_ptr(), pw, sh)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        ms_pp = timed(pool_pass)
        ms_pt = timed(pooled_topk)
        # a decode loop keeps the block keys up to date as blocks fill, so only prefill
        # pays the pooling pass with its selection
        ms_sel = ms_pt if wl.T == 1 else ms_pp + ms_pt
        indexpool = {"pool": pool, "k_blocks": kb, "pool_keys_ms": round(ms_pp, 4),
                     "topk_pooled_ms": round(ms_pt, 4), "token_selection_ms": round(t_topk, 4),
                     "selection_speedup": round(t_topk / ms_sel, 3),
                     "group_step_ms_estimate": round(ms_sel + L * t_attn, 3)}
        del kpool, pws, idx_p

    # ---------------------------------------------------------------- attention backward
    # Gradients of one layer's attention over the same selection (the training side).
    backward = None
    if not args.no_backward and not args.no_extras:
        Lr = layers[0]
        lse0 = torch.empty((wl.B, wl.T, wl.H_q), dtype=torch.float32, device=dev)
        bd.sparse_attn_fwd(qp[0], kp[0], vp[0], idx.data_ptr(), ind["kv_len"].data_ptr(), wl.B,
                           wl.T, wl.S, wl.H_q, wl.H_kv, wl.d, wl.k, wl.sm_scale, op[0],
                           lse0.data_ptr(), ws.data_ptr() if attn_ws else 0, attn_ws, sh)
        dout = torch.randn_like(Lr["q"], dtype=torch.float32).to(torch.bfloat16)
        dq = torch.empty((wl.B, wl.T, wl.H_q, wl.d), dtype=torch.float32, device=dev)
        dK = torch.zeros((wl.B, wl.S, wl.H_kv, wl.d), dtype=torch.float32, device=dev)
        dV = torch.zeros_like(dK)

        # three forms: fp32 atomics (no workspace), and the atomic-free one (inverted
        # selection, per-pair rows, key-major sums) with bf16 or fp32 pair rows, in passes that
        # fit a 32 GiB workspace
        def pass_plan(pair_rows):
            def need(rows):
                return bd.sparse_attn_bwd_workspace_bytes(wl.B, wl.T, wl.S, wl.H_kv, wl.d, wl.k,
                                                          rows, pair_rows)
            rows = int(max(1, min(wl.B * wl.T, (32 << 30) // max(need(2) - need(1), 1))))
            return rows, need(rows)
        plans = {pr: pass_plan(pr) for pr in (bd.PAIR_ROWS_BF16, bd.PAIR_ROWS_FP32)}
        rows_pp, bws_n = plans[bd.PAIR_ROWS_BF16]
        bws = torch.empty(max(n for _, n in plans.values()), dtype=torch.uint8, device=dev)

        def bwd(use_ws, pair_rows=bd.PAIR_ROWS_BF16):
            n = plans[pair_rows][1]
            bd.sparse_attn_bwd(qp[0], kp[0], vp[0], idx.data_ptr(), ind["kv_len"].data_ptr(),
                               op[0], lse0.data_ptr(), dout.data_ptr(), wl.B, wl.T, wl.S, wl.H_q,
                               wl.H_kv, wl.d, wl.k, wl.sm_scale, dq.data_ptr(), dK.data_ptr(),
                               dV.data_ptr(), pair_rows, bws.data_ptr() if use_ws else 0,
                               n if use_ws else 0, sh)
        nb = max(2, min(reps, 5))
        ms_form = {}
        for form in ("atomics", "bf16", "fp32"):
            use_ws = form != "atomics"
            pr = bd.PAIR_ROWS_FP32 if form == "fp32" else bd.PAIR_ROWS_BF16
            bwd(use_ws, pr)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(nb):
                bwd(use_ws, pr)
            e1.record(stream)
            torch.cuda.synchronize()
            ms_form[form] = e0.elapsed_time(e1) / nb
        # IndexShare group: the L layers' backward with the selection inverted once per pass
        # (layer 0's inputs stand in for every layer: the same work per layer)
        ms_group = None
        if L > 1:
            def gbwd():
                bd.indexshare_group_bwd(idx.data_ptr(), ind["kv_len"].data_ptr(), L, [qp[0]] * L,
                                        [kp[0]] * L, [vp[0]] * L, [op[0]] * L,
                                        [lse0.data_ptr()] * L, [dout.data_ptr()] * L, wl.B, wl.T,
                                        wl.S, wl.H_q, wl.H_kv, wl.d, wl.k, wl.sm_scale,
                                        [dq.data_ptr()] * L, [dK.data_ptr()] * L,
                                        [dV.data_ptr()] * L, bd.PAIR_ROWS_BF16, bws.data_ptr(),
                                        bws_n, sh)
            gbwd()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(nb):
                gbwd()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_group = e0.elapsed_time(e1) / nb
        del bws
        ms_b = ms_form["atomics"]
        bflops = sel * 10.0 * wl.H_q * wl.d   # S, dP, dq, dK, dV: 2 H_q d flop each per pair
        backward = {"ms_per_layer": round(min(ms_form.values()), 3),
                    "ms_per_layer_atomics": round(ms_form["atomics"], 3),
                    "ms_per_layer_atomic_free": round(ms_form["bf16"], 3),
                    "atomic_free_rows_per_pass": rows_pp,
                    "ms_per_layer_atomic_free_fp32_rows": round(ms_form["fp32"], 3),
                    "atomic_free_fp32_rows_per_pass": plans[bd.PAIR_ROWS_FP32][0],
                    "group_ms_per_layer_atomic_free": (round(ms_group / L, 3)
                                                       if ms_group is not None else None),
                    # rates of the faster form; the atomic rates below are the atomic form's
                    "bf16_tflops": round(bflops / (min(ms_form.values()) / 1e3) / 1e12, 2),
                    "gathered_GB_per_s": round(sel * 2.0 * wl.d * 2 * wl.H_kv /
                                               (min(ms_form.values()) / 1e3) / 1e9, 1),
                    "fp32_atomic_adds": int(sel * 2 * wl.H_kv * wl.d)}
        del dout, dq, dK, dV

        # fp32 atomic ceiling for that accumulation: 128-float rows added at uniformly random
        # rows of a table the size of dK, one row per wave step (ix_peak_atomic_add)
        rows_tab = wl.B * wl.S * wl.H_kv
        if rows_tab <= (1 << 24):
            tab = torch.zeros(rows_tab * 128, dtype=torch.float32, device=dev)
            n_at = 1 << 22
            rr = torch.randint(0, rows_tab, (n_at,), dtype=torch.int32,
                               generator=torch.Generator(device="cpu").manual_seed(79)).to(dev)
            pk.ix_peak_atomic_add(tab.data_ptr(), rows_tab, rr.data_ptr(), n_at, sh)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(3):
                pk.ix_peak_atomic_add(tab.data_ptr(), rows_tab, rr.data_ptr(), n_at, sh)
            e1.record(stream)
            torch.cuda.synchronize()
            t_at = e0.elapsed_time(e1) / 3 / 1e3
            peak_rate = n_at * 128 / t_at
            backward["fp32_atomic_adds_per_s_measured_peak"] = round(peak_rate / 1e9, 1)
            backward["fp32_atomic_adds_per_s"] = round(sel * 2 * wl.H_kv * wl.d / (ms_b / 1e3) / 1e9, 1)
            backward["frac_of_atomic_peak"] = round(backward["fp32_atomic_adds_per_s"] * 1e9 / peak_rate, 3)
            del tab, rr

        # the indexer's KL objective over the same selection: the kept scores come from
        # ix_topk, the attention normalisers from the forward above
        sel_sc = torch.empty((wl.B, wl.T, wl.k), dtype=torch.float32, device=dev)
        bd.ix_topk(a, wl.k, idx.data_ptr(), sel_sc.data_ptr(), ws.data_ptr(), topk_ws, sh)
        kl_loss = torch.empty((wl.B, wl.T), dtype=torch.float32, device=dev)
        kl_dsc = torch.empty_like(sel_sc)

        def kl():
            bd.ix_indexer_kl(qp[0], kp[0], idx.data_ptr(), ind["kv_len"].data_ptr(),
                             lse0.data_ptr(), sel_sc.data_ptr(), wl.B, wl.T, wl.S, wl.H_q,
                             wl.H_kv, wl.d, wl.k, wl.sm_scale, kl_loss.data_ptr(),
                             kl_dsc.data_ptr(), sh)
        kl()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(nb):
            kl()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_kl = e0.elapsed_time(e1) / nb
        backward["indexer_kl"] = {
            "ms_per_layer": round(ms_kl, 3),
            "bf16_tflops": round(sel * 2.0 * wl.H_q * wl.d / (ms_kl / 1e3) / 1e12, 2),
            "gathered_GB_per_s": round(sel * wl.d * 2 * wl.H_kv / (ms_kl / 1e3) / 1e9, 1)}

        # the KL's score gradient carried into the indexer's inputs (once per group: the
        # layers share the indexer); dk_I accumulates over the reps, which changes no timing
        dq_I = torch.empty((wl.B, wl.T, wl.H_I, wl.d_I), dtype=torch.float32, device=dev)
        dw_I = torch.empty((wl.B, wl.T, wl.H_I), dtype=torch.float32, device=dev)
        dk_I = torch.zeros((wl.B, wl.S, wl.d_I), dtype=torch.float32, device=dev)

        # the forms, as for the attention: atomics, and atomic-free within 32 GiB with bf16 or
        # fp32 pair rows
        def ipass_plan(pair_rows):
            def need(rows):
                return bd.ix_indexer_bwd_workspace_bytes(a, wl.k, rows, pair_rows)
            rows = int(max(1, min(wl.B * wl.T, (32 << 30) // max(need(2) - need(1), 1))))
            return rows, need(rows)
        iplans = {pr: ipass_plan(pr) for pr in (bd.PAIR_ROWS_BF16, bd.PAIR_ROWS_FP32)}
        rows_i = iplans[bd.PAIR_ROWS_BF16][0]
        iws = torch.empty(max(n for _, n in iplans.values()), dtype=torch.uint8, device=dev)

        def ibwd(use_ws, pair_rows=bd.PAIR_ROWS_BF16):
            iws_n = iplans[pair_rows][1]
            bd.ix_indexer_bwd(a, wl.k, idx.data_ptr(), kl_dsc.data_ptr(), dq_I.data_ptr(),
                              dw_I.data_ptr(), dk_I.data_ptr(), pair_rows,
                              iws.data_ptr() if use_ws else 0, iws_n if use_ws else 0, sh)
        ms_iform = {}
        for form in ("atomics", "bf16", "fp32"):
            use_ws = form != "atomics"
            pr = bd.PAIR_ROWS_FP32 if form == "fp32" else bd.PAIR_ROWS_BF16
            ibwd(use_ws, pr)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(nb):
                ibwd(use_ws, pr)
            e1.record(stream)
            torch.cuda.synchronize()
            ms_iform[form] = e0.elapsed_time(e1) / nb
        del iws
        ms_ib = ms_iform["atomics"]
        adds = sel * wl.d_I
        backward["indexer_backward"] = {
            "ms_per_group": round(min(ms_iform.values()), 3),
            "ms_per_group_atomics": round(ms_iform["atomics"], 3),
            "ms_per_group_atomic_free": round(ms_iform["bf16"], 3),
            "atomic_free_rows_per_pass": rows_i,
            "ms_per_group_atomic_free_fp32_rows": round(ms_iform["fp32"], 3),
            "atomic_free_fp32_rows_per_pass": iplans[bd.PAIR_ROWS_FP32][0],
            "mfma_tflops": round(sel * 6.0 * wl.H_I * wl.d_I / (ms_ib / 1e3) / 1e12, 2),
            "fp32_atomic_adds": int(adds),
            "fp32_atomic_adds_per_s": round(adds / (ms_ib / 1e3) / 1e9, 1)}
        if "fp32_atomic_adds_per_s_measured_peak" in backward:
            backward["indexer_backward"]["frac_of_atomic_peak"] = round(
                adds / (ms_ib / 1e3) / 1e9 / backward["fp32_atomic_adds_per_s_measured_peak"], 3)
        del lse0, sel_sc, kl_loss, kl_dsc, dq_I, dw_I, dk_I

    # ---------------------------------------------------------------- per-layer indexing
    indexshare = None
    if not args.no_per_layer and L > 1:
        inds = [ind] + [synth.indexer_inputs(wl, layer=l, device=dev) for l in range(1, L)]
        aa = [bd.indexer_args(x["q_I"], x["k_I"], x["w"], x["q_pos0"], x["kv_len"]) for x in inds]

        def per_layer_step():
            for l in range(L):
                bd.ix_topk(aa[l], wl.k, idx.data_ptr(), 0, ws.data_ptr(), topk_ws, sh)
                bd.sparse_attn_fwd(qp[l], kp[l], vp[l], idx.data_ptr(),
                                   inds[l]["kv_len"].data_ptr(), wl.B, wl.T, wl.S, wl.H_q,
                                   wl.H_kv, wl.d, wl.k, wl.sm_scale, op[l], 0,
                                   ws.data_ptr() if attn_ws else 0, attn_ws, sh)
        per_layer_step()
        torch.cuda.synchronize()
        n_pl = max(2, args.steps // 2)
        e0.record(stream)
        for _ in range(n_pl):
            per_layer_step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_pl = e0.elapsed_time(e1) / n_pl
        indexshare = {"group_ms": round(ms, 3), "per_layer_ms": round(ms_pl, 3),
                      "speedup": round(ms_pl / ms, 3), "layers": L}
        del inds, aa

    # ---------------------------------------------------------------- measured ceilings
    peaks = None
    if not args.no_peaks and not args.no_extras:
        peaks = measured_peaks(dev, sh, codes=torch.cat([ind["k_I"].reshape(-1)[:1 << 20],
                                                          ind["q_I"].reshape(-1)[:1 << 20]]))
        if idx_roof["bound"] == "mfma":
            by_valu = peaks["fp8_mfma_tflops_by_valu_per_mfma"]
            # the plain epilogue's ceiling (8 VALU ops per MFMA), and that of the 64-head
            # |x| + linear-MFMA form: about 4-5 VALU ops per MFMA, 16 of every 17 MFMAs useful
            peaks["indexer_frac_of_mfma_with_8_valu"] = round(idx_roof["achieved"] / by_valu["8"], 3)
            peaks["indexer_frac_of_mfma_with_4_valu_16_of_17"] = round(
                idx_roof["achieved"] / (by_valu["4"] * 16 / 17), 3)
        else:
            peaks["indexer_frac_of_read"] = round(idx_roof["achieved"] / peaks["read_GB_per_s"], 3)
        peaks["attention_frac_of_gather_64MiB"] = round(
            attn_roof["achieved"] / peaks["gather_256B_rows_GB_per_s"]["64MiB"], 3)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wl, name, ind, layers, dev)

    # ---------------------------------------------------------------- decode and 1M legs
    legs = {}
    if not args.no_legs and not args.no_extras:
        del ind, layers, outs, ws, idx, a
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for leg_name in ("decode_b64_128k", "chunk_prefill_1m"):
            if leg_name != name:
                legs[leg_name] = run_leg(leg_name, dev, args.steps)
    gather_hbm = None
    if "decode_b64_128k" in legs:
        d = legs["decode_b64_128k"]
        gather_hbm = {"workload": "decode_b64_128k",
                      "kernel": "sparse_attn_group_fwd: the 4 layers' attention of the decode "
                                "step in one launch, caches flushed, issued straight after "
                                "the flush",
                      "bound": "hbm", "achieved": d["group_attention_GB_per_s_cold_back_to_back"],
                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": d["group_attention_hbm_frac_cold_back_to_back"],
                      "ms_per_layer": d["group_attention_ms_per_layer_cold_back_to_back"],
                      "per_call": {"ms_per_layer": d["group_attention_ms_per_layer_cold"],
                                   "frac": d["group_attention_hbm_frac_cold"],
                                   "note": "events around each call: adds the dispatch gap"},
                      "one_layer_call": {"ms": d["attention_ms_per_layer_cold_back_to_back"],
                                         "frac": d["attention_hbm_frac_cold_back_to_back"],
                                         "ms_per_call_timed": d["attention_ms_per_layer_cold"],
                                         "gather_ceiling": d["gather_ceiling_cold"]}}
    if "decode_b64_128k" in legs and peaks:
        d = legs["decode_b64_128k"]
        rate = d["indexer_bytes"] / (d["ix_topk_ms"] / 1e3) / 1e9
        d["indexer_GB_per_s"] = round(rate, 1)
        d["indexer_frac_of_read_ceiling"] = round(rate / peaks["read_GB_per_s"], 4)
        d["indexer_frac_of_read_ceiling_cold"] = round(
            d["indexer_bytes"] / (d["ix_topk_ms_cold"] / 1e3) / 1e9 / peaks["read_GB_per_s"], 4)
        # against the stream at the sweep's own occupancy (the best grid has 2-4x the waves)
        d["indexer_frac_of_read_at_1024_waves"] = round(rate / peaks["read_GB_per_s_1024_waves"], 4)
        if gather_hbm:
            g = peaks["gather_256B_rows_GB_per_s"]
            ceil = g.get("16GiB", g["2GiB"])
            gather_hbm["random_gather_ceiling"] = {
                "GB_per_s": ceil, "footprint": "16GiB" if "16GiB" in g else "2GiB",
                "note": "random 256-byte rows over the decode step's 4 layers of K and V"}
            gather_hbm["frac_of_random_gather_ceiling"] = round(gather_hbm["achieved"] / ceil, 4)
    indexshare_1m = None
    if "chunk_prefill_1m" in legs:
        c = legs["chunk_prefill_1m"]
        n_l, fi, fa = c["layers"], c["indexer_tflop"], c["attention_tflop_per_layer"]
        indexshare_1m = {"workload": "chunk_prefill_1m", "group_ms": c["group_ms"],
                         "per_layer_indexing_ms": c["per_layer_indexing_ms"],
                         "speedup": c["indexshare_speedup"], "target": 2.0,
                         # this path's flops: one indexer per group against one per layer
                         "path_flop_ratio": round((n_l * fi + n_l * fa) / (fi + n_l * fa), 3),
                         "pages_claim": "2.9x fewer FLOPs per token at 1M context (the pages' "
                                        "figure for the whole model, with no hardware or timing; "
                                        "context only)"}

    line = {
        "metric": "query tokens/s (indexer+topk+sparse attn) at 128K; FP8 MFMA % and HBM % of peak",
        "value": round(value, 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": name, "B": wl.B, "T": wl.T, "S": wl.S, "H_I": wl.H_I,
                   "d_I": wl.d_I, "k": wl.k, "H_q": wl.H_q, "H_kv": wl.H_kv, "d": wl.d,
                   "layers": L, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gather_hbm_128k": gather_hbm,
        "indexshare_1m": indexshare_1m,
        "detail": {
            "ix_topk_ms": round(t_topk, 3),
            "sparse_attn_ms_per_layer": round(t_attn, 3),
            "ix_topk_ms_median": round(float(np.median(topk_times)), 3),
            "sparse_attn_ms_per_layer_median": round(float(np.median(attn_times)), 3),
            "per_kernel_reps": reps,
            "indexer_roofline": idx_roof,
            "attention_roofline": attn_roof,
            "indexer_tflop": round(flops / 1e12, 3),
            "attention_gb_per_layer": round(attn_bytes / 1e9, 3),
            "visible_pairs": pairs,
            "selected_pairs": sel,
            "indexshare": indexshare,
            "cache_append": append,
            "indexpool": indexpool,
            "attention_backward": backward,
            "attention_cold": attn_cold,
            "measured_peaks": peaks,
            "legs": legs,
            "wall_s_timed_region": round(t_wall, 3),
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
