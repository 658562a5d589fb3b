"""Turn rocprofv3 CSV output into the short summaries kept under ``profiles/``.

Commands (run on the CSV files a GPU run wrote):

  python -m paged_kv_cache_reshape_amd.profiling trace KERNEL_STATS_CSV OUT_MD \\
      --command "<the rocprofv3 command that produced it>"

  python -m paged_kv_cache_reshape_amd.profiling traffic FETCH_CSV WRITE_CSV \\
      --workload qwen3_0p6b --partition-size 1024 --command "<...>"

  python -m paged_kv_cache_reshape_amd.profiling counters OUT_MD --kernel NAME \\
      --command "<...>" COUNTER_CSV [COUNTER_CSV ...]

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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _kernel_key(name: str) -> str:
    if "decode_partition_kernel" in name or "decode_mfma_kernel" in name:
        return "decode"
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
            k = f"copy grid={r['Grid_Size']}"
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
    # The biggest copy kernel clones one K cache: k_cache_bytes read and written.
    copy_key = max((k for k in fetch if k.startswith("copy")), key=lambda k: fetch[k])
    fetch_factor = k_cache_bytes / 1024.0 / fetch[copy_key]
    write_factor = k_cache_bytes / 1024.0 / write[copy_key]
    # WRITE_SIZE reads a clone's bytes exactly; far from that, the run made no
    # clone (a pool too large to replicate keeps one copy) and the counters
    # have nothing of known size to be scaled by.
    if not 0.9 <= write_factor <= 1.1:
        raise ValueError(f"the largest copy kernel wrote {write[copy_key]:.1f} KiB, not one "
                         f"K cache ({k_cache_bytes / 1024.0:.1f} KiB): no clone to scale by")
    read_b = fetch["decode"] * fetch_factor * 1024.0
    write_b = write["decode"] * write_factor * 1024.0
    # Counters of a `bench.py --step-only` run see only the fused step's
    # launches (decode with the KV write in it): their algorithmic bytes.
    inp_bytes = bench.algorithmic_bytes(synth.make_inputs(w))["step" if fused_step else "decode"]
    out_json = bench.traffic_file(workload)
    rec = {
        "workload": workload,
        "partition_size": partition_size,
        "kernel": bench.decode_kernel_name(w),
        "launch": "fused step" if fused_step else "decode",
        "command": command,
        "fetch_size_kib_per_dispatch": round(fetch["decode"], 2),
        "write_size_kib_per_dispatch": round(write["decode"], 2),
        "copy_kernel_bytes": k_cache_bytes,
        "copy_fetch_size_kib": round(fetch[copy_key], 2),
        "copy_write_size_kib": round(write[copy_key], 2),
        "fetch_scale": round(fetch_factor, 5),
        "write_scale": round(write_factor, 5),
        "hbm_read_bytes_per_launch": int(read_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(read_b + write_b),
        "algorithmic_bytes_per_launch": inp_bytes,
        "traffic_over_algorithmic": round((read_b + write_b) / inp_bytes, 4),
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
        f"| copy kernel, {k_cache_bytes} B known | {fetch[copy_key]:.1f} | {write[copy_key]:.1f} |\n"
        f"| scale (known / counter) | {fetch_factor:.5f} | {write_factor:.5f} |\n"
        f"| decode kernel | {fetch['decode']:.1f} | {write['decode']:.1f} |\n\n"
        f"Decode HBM bytes per launch: read {read_b / 1e6:.2f} MB + written "
        f"{write_b / 1e6:.3f} MB = {(read_b + write_b) / 1e6:.2f} MB; algorithmic "
        f"{inp_bytes / 1e6:.2f} MB (ratio {(read_b + write_b) / inp_bytes:.4f}).\n")
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
    c = sub.add_parser("counters")
    c.add_argument("out_md")
    c.add_argument("csvs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        trace_summary(a.stats_csv, a.out_md, a.command)
    elif a.cmd == "counters":
        print(json.dumps(counters_summary(a.csvs, a.kernel, a.out_md, a.command), indent=1))
    else:
        print(json.dumps(traffic_record(a.fetch_csv, a.write_csv, a.workload,
                                        a.partition_size, a.command, a.fused_step), indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
