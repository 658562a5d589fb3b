"""Turn rocprofv3 CSV output into the short summaries kept under ``profiles/``.

Commands (run on the CSV files a GPU run wrote):

  python profiling.py trace KERNEL_STATS_CSV OUT_MD \\
      --command "<the rocprofv3 command that produced it>"

  python profiling.py traffic FETCH_CSV WRITE_CSV \\
      --workload qwen3_0p6b --partition-size 1024 --command "<...>"

  python profiling.py counters OUT_MD --kernel NAME \\
      --command "<...>" COUNTER_CSV [COUNTER_CSV ...]

  python profiling.py timeline BENCH_TIMELINE_JSON OUT_MD --command "<...>"

``traffic`` scales the per-dispatch FETCH_SIZE and WRITE_SIZE of the decode
kernel by what the same counters read for the plain copy kernels in the same
run (PyTorch cloning one K cache, a copy of known size), and records the hash
of the decode kernel's sources so that ``bench.py`` reports the figure only
while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _kernel_key(name: str) -> str:
    if ("decode_partition_kernel" in name or "decode_mfma_kernel" in name
            or "decode_stream_kernel" in name or "decode_stream_mfma_kernel" in name):
        return "decode"
    if "merge_partitions_kernel" in name or "stream_merge_kernel" in name:
        return "merge"
    if "kv_write_kernel" in name:
        return "kv_write"
    if "copyBuffer" in name:
        return "copy"
    return name[:60]


def trace_summary(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel trace summary", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.3f} | {float(r['MinNs']) / 1e3:.3f} | "
                     f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f}% |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_dispatch(counter_csv: str, counter: str) -> dict:
    agg = collections.defaultdict(list)
    grids = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        k = _kernel_key(r["Kernel_Name"])
        if k == "copy":
            # Each copy on its own: copies of different sizes share a grid.
            k = f"copy dispatch {r.get('Dispatch_Id', len(grids))}"
            grids[k] = int(r["Grid_Size"])
        agg[k].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic_record(fetch_csv: str, write_csv: str, workload: str, partition_size: int,
                   command: str, fused_step: bool = False) -> dict:
    import numpy as np

    import bench
    import synth

    w = synth.WORKLOADS[workload]
    ctx = synth.draw_context_lens(w, np.random.default_rng(w.seed))
    k_cache_bytes = (synth.pool_blocks(w, ctx) * w.block_size * w.num_kv_heads *
                     w.head_dim * w.elt_bytes)
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    # Copies of known size in the run: the calibration clone `bench.py
    # --step-only` makes (bench.CALIBRATION_BYTES) and the clones of one K
    # cache that replicate the pool.  WRITE_SIZE reads a clone's bytes almost
    # exactly, which tells the copies apart; the largest one found fixes the
    # scale of each counter.
    # The two runs make the same dispatches in the same order, so a copy's
    # dispatch id names it in both.
    known = {}
    for k in fetch:
        if not k.startswith("copy") or k not in write or write[k] <= 0:
            continue
        for size in (bench.CALIBRATION_BYTES, k_cache_bytes):
            if 0.9 <= size / 1024.0 / write[k] <= 1.1:
                known.setdefault(size, []).append(k)
    if not known:
        raise ValueError("no copy kernel wrote a known size (the calibration clone of "
                         f"{bench.CALIBRATION_BYTES} B or one K cache of {k_cache_bytes} B): "
                         "no clone to scale by")
    copy_bytes = max(known)
    keys = known[copy_bytes]
    copy_fetch = sum(fetch[k] for k in keys) / len(keys)
    copy_write = sum(write[k] for k in keys) / len(keys)
    fetch_factor = copy_bytes / 1024.0 / copy_fetch
    write_factor = copy_bytes / 1024.0 / copy_write
    read_b = fetch["decode"] * fetch_factor * 1024.0
    write_b = write["decode"] * write_factor * 1024.0
    # A separate merge kernel (a launch of its own after the decode when a
    # sequence has many partitions) is reported beside the decode kernel.
    merge_b = ((fetch.get("merge", 0.0) * fetch_factor + write.get("merge", 0.0) * write_factor)
               * 1024.0)
    # Counters of a `bench.py --step-only` run see only the fused step's
    # launches (decode with the KV write in it): their algorithmic bytes.
    inp_bytes = bench.algorithmic_bytes(synth.make_inputs(w))["step" if fused_step else "decode"]
    out_json = bench.traffic_file(workload)
    rec = {
        "workload": workload,
        "partition_size": partition_size,
        "kernel": bench.decode_kernel_name(w, partition_size),
        "launch": "fused step" if fused_step else "decode",
        "command": command,
        "fetch_size_kib_per_dispatch": round(fetch["decode"], 2),
        "write_size_kib_per_dispatch": round(write["decode"], 2),
        "copy_kernel_bytes": copy_bytes,
        "copy_fetch_size_kib": round(copy_fetch, 2),
        "copy_write_size_kib": round(copy_write, 2),
        "copy_dispatches": len(keys),
        "fetch_scale": round(fetch_factor, 5),
        "write_scale": round(write_factor, 5),
        "hbm_read_bytes_per_launch": int(read_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "algorithmic_bytes_per_launch": inp_bytes,
        "traffic_over_algorithmic": round((read_b + write_b) / inp_bytes, 4),
        "merge_kernel_bytes_per_launch": int(merge_b) if "merge" in fetch else None,
        "kernel_source_sha256": bench.kernel_source_hash(),
    }
    json.dump(rec, open(out_json, "w"), indent=1)
    md = os.path.splitext(out_json)[0] + ".md"
    open(md, "w").write(
        f"# HBM traffic of {rec['kernel']}\n\n"
        f"Workload `{workload}`, partition size {partition_size}; "
        f"{'launches of the fused step (the KV write inside the decode)' if fused_step else 'decode launches'}.\n\n"
        "Commands (one counter per run):\n\n```\n" + command + "\n```\n\n"
        "| | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) |\n|---|---|---|\n"
        f"| copy kernel, {copy_bytes} B known ({len(keys)} dispatches) | {copy_fetch:.1f} | "
        f"{copy_write:.1f} |\n"
        f"| scale (known / counter) | {fetch_factor:.5f} | {write_factor:.5f} |\n"
        f"| decode kernel | {fetch['decode']:.1f} | {write['decode']:.1f} |\n\n"
        f"Decode HBM bytes per launch: read {read_b / 1e6:.2f} MB + written "
        f"{write_b / 1e6:.3f} MB = {(read_b + write_b) / 1e6:.2f} MB; algorithmic "
        f"{inp_bytes / 1e6:.2f} MB (ratio {(read_b + write_b) / inp_bytes:.4f}).\n"
        + (f"\nSeparate merge kernel (its own launch after each decode): "
           f"{merge_b / 1e6:.3f} MB per launch.\n" if "merge" in fetch else ""))
    return rec


def counters_summary(csvs: list, kernel: str, out_md: str, command: str) -> dict:
    """Average per dispatch of every counter collected for the kernels whose
    name contains `kernel`, over one or more counter-collection CSVs (one
    rocprofv3 --pmc pass each)."""
    agg = collections.defaultdict(list)
    for path in csvs:
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                agg[r["Counter_Name"]].append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in sorted(agg.items())}
    lines = [f"# Hardware counters of `{kernel}`", "", "Commands (one pass each):", "", "```",
             command, "```", "", "| counter | average per dispatch | dispatches |",
             "|---|---|---|"]
    for k, v in avg.items():
        lines.append(f"| {k} | {v:.6g} | {len(agg[k])} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    return avg


def timeline_md(bench_json: str, out_md: str, command: str) -> None:
    """The per-wave timeline that ``bench.py --timeline`` printed, as a short
    markdown summary."""
    res = json.loads(open(bench_json).read().strip().splitlines()[-1])
    t = res["timeline"]
    lines = [f"# Per-wave timeline of the stream kernel, {res['config']['workload'].split(':')[0]}",
             "", "Command:", "", "```", command, "```", "",
             f"Step time in the same run (measurement build): {res['us_per_step']} us; "
             f"{t['waves']} worker waves, {t['mergers']} of them merge a split sequence; "
             f"constant clock {t['clock_khz']} kHz. Offsets from the first wave's start (us):",
             "", "| event | median | p90 | max |", "|---|---|---|---|",
             f"| wave start | | | {t['start_us']['max']} |",
             *([f"| lengths read and prefix-summed | {t['lengths_end_us']['median']} | | "
                f"{t['lengths_end_us']['max']} |"] if t.get("lengths_end_us") else []),
             *([f"| range's table entries requested | {t['range_end_us']['median']} | | "
                f"{t['range_end_us']['max']} |"] if t.get("range_end_us") else []),
             f"| first block requested (prologue end) | {t['prologue_end_us']['median']} | "
             f"{t['prologue_end_us']['p90']} | {t['prologue_end_us']['max']} |",
             f"| range streamed (stream end) | {t['stream_end_us']['median']} | "
             f"{t['stream_end_us']['p90']} | {t['stream_end_us']['max']} |",
             f"| done | | | {t['done_us_max']} |", "",
             f"Earliest stream end: {t['stream_end_us']['min']} us. Latest stream end per XCD: "
             f"{', '.join(str(x) for x in t['stream_end_us_per_xcd_max'])} us."]
    if t.get("merge_us"):
        lines.append(f"Merge (stream end to done, merging waves): median {t['merge_us']['median']}"
                     f" us, max {t['merge_us']['max']} us.")
    if t.get("compute_units"):
        hosted = ", ".join(f"{n} CUs with {k} waves" for k, n in t["cus_by_waves_hosted"].items())
        ce = t["cu_stream_end_us"]
        lines.append(f"Compute units used: {t['compute_units']} ({hosted}). Latest stream end per "
                     f"CU: min {ce['min']}, median {ce['median']}, max {ce['max']} us.")
    lw = t["last_wave"]
    lines.append(f"The last wave to finish ended its stream at {lw['stream_end_us']} us and was "
                 f"done at {lw['done_us']} us ({'a merger' if lw['merger'] else 'not a merger'}); "
                 f"the last stream end to the last wave done: {t['last_stream_end_to_done_us']} us.")
    open(out_md, "w").write("\n".join(lines) + "\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_md")
    t.add_argument("--command", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("fetch_csv")
    f.add_argument("write_csv")
    f.add_argument("--workload", default="qwen3_0p6b")
    f.add_argument("--partition-size", type=int, required=True)
    f.add_argument("--command", required=True)
    f.add_argument("--fused-step", action="store_true",
                   help="the counters come from `bench.py --step-only` (fused-step launches)")
    tl = sub.add_parser("timeline")
    tl.add_argument("bench_json")
    tl.add_argument("out_md")
    tl.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out_md")
    c.add_argument("csvs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        trace_summary(a.stats_csv, a.out_md, a.command)
    elif a.cmd == "timeline":
        timeline_md(a.bench_json, a.out_md, a.command)
    elif a.cmd == "counters":
        print(json.dumps(counters_summary(a.csvs, a.kernel, a.out_md, a.command), indent=1))
    else:
        print(json.dumps(traffic_record(a.fetch_csv, a.write_csv, a.workload,
                                        a.partition_size, a.command, a.fused_step), indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
