"""Host-side tools of the benchmark, checked without a GPU: the algorithmic
byte counts the roofline divides by, and the HBM-traffic record built from
rocprofv3 counter files (scaled by a copy kernel of known size)."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth
import profiling


def test_algorithmic_bytes_of_the_tiny_batch():
    """Worked by hand: contexts {1, 17, 33, 64} (115 tokens), B=4, Hq=4,
    Hkv=2, D=64, 4-byte elements, 16-token blocks."""
    nb = bench.algorithmic_bytes(synth.make_inputs(synth.WORKLOADS["tiny_f32"]))
    assert nb["kv"] == 115 * 2 * 2 * 64 * 4 == 117_760      # K and V rows read once
    q_and_out = 2 * 4 * 4 * 64 * 4                          # q read, out written
    table = (1 + 2 + 3 + 4) * 4 + 4 * 4                     # used entries + lengths
    assert nb["decode"] == nb["kv"] + q_and_out + table
    write = 2 * 2 * 4 * 2 * 64 * 4 + 8 * 4                  # 4 new K/V rows in and out, slots
    assert nb["write"] == write
    assert nb["step"] == nb["decode"] + nb["write"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                           "Grid_Size"])
        wr.writeheader()
        for name, value, grid in rows:
            wr.writerow(dict(Kernel_Name=name, Counter_Name=counter, Counter_Value=value,
                             Grid_Size=grid))


@pytest.mark.parametrize("fused", [False, True])
def test_traffic_record_is_scaled_by_the_copy_kernel(tmp_path, monkeypatch, fused):
    """The biggest copy kernel clones one K pool (size known): its counter
    readings fix the scale of each counter; the decode kernel's mean reading
    per dispatch, so scaled, is the record's HBM bytes per launch, set
    against the step's algorithmic bytes for fused-step counter runs and the
    decode's otherwise."""
    wl = "tiny_f32"
    w = synth.WORKLOADS[wl]
    ctx = synth.draw_context_lens(w, np.random.default_rng(w.seed))
    k_bytes = (synth.pool_blocks(w, ctx) * w.block_size * w.num_kv_heads * w.head_dim *
               w.elt_bytes)
    dec = "void pa::decode_partition_kernel<pa::F32, 64, 16, 2, 4>(pa::DecodeArgs)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # FETCH_SIZE reads half of what the copy moved, WRITE_SIZE all of it (KiB).
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", k_bytes / 2048, 999),
                                       ("__amd_rocclr_copyBuffer", 1.0, 3),
                                       (dec, 100.0, 64), (dec, 140.0, 64)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", k_bytes / 1024, 999),
                                       ("__amd_rocclr_copyBuffer", 1.0, 3),
                                       (dec, 2.0, 64), (dec, 4.0, 64)])
    monkeypatch.setattr(bench, "traffic_file",
                        lambda workload: str(tmp_path / f"traffic_{workload}.json"))
    rec = profiling.traffic_record(str(fetch), str(write), wl, 512, "the commands", fused)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_read_bytes_per_launch"] == 120 * 2 * 1024
    assert rec["hbm_write_bytes_per_launch"] == 3 * 1024
    nb = bench.algorithmic_bytes(synth.make_inputs(w))
    assert rec["algorithmic_bytes_per_launch"] == nb["step" if fused else "decode"]
    assert rec["launch"] == ("fused step" if fused else "decode")
    # Written where the benchmark looks, under the current source hash, so
    # the benchmark takes it; another hash makes it stale.
    assert bench.traffic_record(wl) == json.load(open(tmp_path / f"traffic_{wl}.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.traffic_record(wl) is None


def test_traffic_record_needs_a_clone_of_known_size(tmp_path, monkeypatch):
    """Without a copy kernel that cloned one K pool (a run that kept a single
    pool copy), the counters cannot be scaled and no record is written."""
    wl = "tiny_f32"
    dec = "void pa::decode_partition_kernel<pa::F32, 64, 16, 2, 4>(pa::DecodeArgs)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1.0, 3), (dec, 100.0, 64)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1.0, 3), (dec, 2.0, 64)])
    monkeypatch.setattr(bench, "traffic_file",
                        lambda workload: str(tmp_path / f"traffic_{workload}.json"))
    with pytest.raises(ValueError, match="no clone"):
        profiling.traffic_record(str(fetch), str(write), wl, 512, "the commands", True)
    assert not os.path.exists(tmp_path / f"traffic_{wl}.json")


def test_traffic_record_takes_the_calibration_copy(tmp_path, monkeypatch):
    """A pool too large to replicate (one copy, no K clone): the calibration
    clone of bench.CALIBRATION_BYTES made in the same run scales the
    counters; a separate merge kernel is reported beside the decode."""
    wl = "tiny_f32"
    cal = bench.CALIBRATION_BYTES
    dec = "void pa::decode_stream_kernel<pa::F32, 64, 16, 2, true>(pa::DecodeArgs)"
    mrg = "void pa::merge_partitions_kernel<pa::F32, 64, 2>(pa::DecodeArgs)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", cal / 4096, 4096),
                                       (dec, 100.0, 64), (mrg, 3.0, 8)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", cal / 1024 * 1.02, 4096),
                                       (dec, 2.0, 64), (mrg, 1.0, 8)])
    monkeypatch.setattr(bench, "traffic_file",
                        lambda workload: str(tmp_path / f"traffic_{workload}.json"))
    rec = profiling.traffic_record(str(fetch), str(write), wl, 0, "the commands", True)
    assert rec["copy_kernel_bytes"] == cal
    assert rec["fetch_scale"] == 4.0
    assert abs(rec["write_scale"] - 1 / 1.02) < 1e-5
    assert rec["hbm_read_bytes_per_launch"] == 400 * 1024
    assert rec["merge_kernel_bytes_per_launch"] == int((3.0 * 4 + 1.0 / 1.02) * 1024)
    assert rec["kernel"] == "decode_stream_kernel"


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: with --gpus 2 the benchmark says so and exits with 2."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_timeline_stats_and_summary(tmp_path):
    """The per-wave timeline summary on hand-made records: four streaming
    waves on two compute units (100 MHz clock, so one tick is 0.01 us), one
    of them a merger, and a copy wave that only stamped its start."""
    def hw(xcc, se, cu):
        return (xcc << 32) | (se << 13) | (cu << 8)
    base = 1_000_000
    rec = np.zeros((8, 6), dtype=np.int64)
    #            start        prologue      stream end     done           ids         merged
    rec[0] = [base,        base + 280,   base + 2400,   base + 2410,   hw(0, 1, 3), 0]
    rec[1] = [base + 10,   base + 300,   base + 2500,   base + 2800,   hw(0, 1, 3), 3]
    rec[2] = [base + 5,    base + 260,   base + 2100,   base + 2105,   hw(1, 0, 7), 0]
    rec[3] = [base + 20,   base + 290,   base + 2600,   base + 2605,   hw(1, 0, 7), 0]
    rec[4] = [base + 30,   0,            0,             0,             hw(1, 0, 2), 0]
    t = bench.timeline_stats(rec, 100_000)
    assert t["waves"] == 4 and t["mergers"] == 1
    assert t["prologue_end_us"]["max"] == 3.0
    assert t["stream_end_us"]["min"] == 21.0 and t["stream_end_us"]["max"] == 26.0
    assert t["done_us_max"] == 28.0
    assert t["merge_us"]["median"] == 3.0
    assert t["last_wave"] == {"stream_end_us": 25.0, "done_us": 28.0, "merger": True}
    assert t["last_stream_end_to_done_us"] == 2.0
    assert t["compute_units"] == 2 and t["cus_by_waves_hosted"] == {2: 2}
    assert t["cu_stream_end_us"]["min"] == 25.0 and t["cu_stream_end_us"]["max"] == 26.0
    j = tmp_path / "tl.json"
    j.write_text(json.dumps({"us_per_step": 31.8, "timeline": t,
                             "config": {"workload": "qwen3_0p6b: B=32"}}) + "\n")
    md = tmp_path / "tl.md"
    profiling.timeline_md(str(j), str(md), "python bench.py --timeline")
    text = md.read_text()
    assert "| range streamed (stream end) |" in text and "2 CUs with 2 waves" in text

