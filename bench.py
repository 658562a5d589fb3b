"""Benchmark of one decode step (paged KV write + paged decode attention) on one GPU.

A step is one pass of the whole path over one synthetic batch: each
sequence's new K/V row is written into the paged caches and the decode runs
over the updated caches, both in one launch (``decode_step``, the write fused
into the decode kernel; the same bits as ``reshape_and_cache`` followed by
``paged_attention_decode``, whose two-launch step is timed too).  Default workload: the Qwen3-0.6B-shaped batch
(B=32, Hq=16, Hkv=8, D=128, block_size=16, context lengths uniform in
[128, 2048], bf16 storage, float32 accumulation).

Inputs are resident in HBM before timing starts.  To keep the timed reads
coming from HBM rather than the 256 MB last-level cache, the step cycles
through R identical copies of the KV pool (>= 1.25 GiB together).

Prints one JSON line.  ``value`` is the step's algorithmic bytes (KV rows
read, q read, output written, block-table entries, the write's rows) divided by
the step time.  ``roofline`` is for the step's kernel (the decode with the
write fused in): its algorithmic bytes per launch over its mean launch time in
the timed region, from HIP events on the stream it runs on around the K
back-to-back steps.  ``decode_us_mean`` times the decode alone the same way,
``unfused_us_per_step`` the two-launch step.  ``graph_us_per_step`` is the
step replayed from a HIP graph.  ``decode_us_loops`` / ``decode_us_median``
are five more loops of decode launches timed one by one; ``mall_resident`` is the
decode reading one warm pool copy every launch; ``cache_line_efficiency`` is
the step's algorithmic bytes over the HBM bytes the counters measured on the
step's launches (a ``--step-only`` run, on the current kernel sources).  ``prior_art`` times the
pages' earlier design on the same GPU (gather the pages into dense tensors,
then ordinary attention, in PyTorch).  ``cpu_baseline`` times the float64 CPU
oracle on a bounded sample of the same batch, spread over the host's cores
and again on one thread.  ``read_ceiling`` times kernels that only read the
decode's K/V bytes, in three access patterns (read_ceiling.hip): the floor
under any decode that reads the cache that way.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode-attention KV GB/s and % of HBM peak; µs/step at B=32 Qwen3-0.6B shape"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_reshape_amd", "csrc", f)
               for f in ("decode_partition.hip", "decode_mfma.hip", "decode_stream.hip",
                         "decode_stream_mfma.hip",
                         "attn_common.hpp", "mfma_attn.hpp", "stream_sched.hpp", "common.hpp",
                         "decode_launch.hpp", "decode_api.hip", "options.hpp", "timeline.hpp")]
# Worker processes the CPU baseline spreads the oracle over: the host's cores,
# at most 16 (one GPU's share of a shared host).
CPU_POOL_MAX = 16
# A copy of known size made in counter runs (--step-only): rocprofv3's
# FETCH_SIZE / WRITE_SIZE of the decode kernel are scaled by what they read
# for this copy.
CALIBRATION_BYTES = 256 << 20


def algorithmic_bytes(inp: dict) -> dict:
    """Bytes the step must move at least once (no re-reads, no partials)."""
    w = inp["workload"]
    ctx = inp["context_lens"].astype(np.int64)
    elt = w.elt_bytes
    kv = int(ctx.sum()) * 2 * w.num_kv_heads * w.head_dim * elt
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * elt
    tables = int(sum(-(-int(c) // w.block_size) for c in ctx)) * 4 + 4 * w.num_seqs
    n_new = int((inp["slot_mapping"] >= 0).sum())
    write = 2 * 2 * n_new * w.num_kv_heads * w.head_dim * elt + 8 * w.num_seqs
    return dict(kv=kv, decode=kv + qo + tables, write=write,
                step=kv + qo + tables + write)


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def traffic_record(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the decode kernels as they are now (source hash
    matches)."""
    try:
        rec = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def kernel_source_hash() -> str:
    """sha256 over the decode kernel's sources, in a fixed order."""
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_kernel_name(w, partition_size: int | None = None) -> str:
    """The decode kernel the library runs for this workload: the balanced
    schedule's kernel when the library reports partition size 0 (its
    matrix-core worker for bfloat16 with 4 query heads per kv head), else the
    matrix-core kernel for bfloat16 with 4, 8, 16 or 32 query heads per kv
    head (4 only over block tables of at most 4096 tokens), the vector-ALU
    kernel otherwise."""
    if partition_size == 0:
        g = w.num_q_heads // w.num_kv_heads
        return ("decode_stream_mfma_kernel" if w.dtype == "bf16" and g == 4
                else "decode_stream_kernel")
    g = w.num_q_heads // w.num_kv_heads
    long_table = w.max_blocks_per_seq * w.block_size > 4096
    mfma = w.dtype == "bf16" and (g in (8, 16, 32) or (g == 4 and not long_table))
    return "decode_mfma_kernel" if mfma else "decode_partition_kernel"


def gather_then_attention(q, k_cache, v_cache, block_tables, context_lens, scale):
    """The pages' prior art on the same GPU, in PyTorch: gather every
    sequence's pages into dense, padded tensors, then ordinary masked
    attention (barellm README, feature list: pages gathered into dense tensors
    for SDPA; MinivLLM article, "What the Two Benchmark Scripts Compare": the
    vectorised PyTorch decode with batch gathering and masking).  The gather
    moves bf16 rows; the attention runs in float32 with contiguous matmul
    operands.  Returns (out [B, Hq, D] in q's dtype, the dense K and V)."""
    import torch
    B, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    g = hq // hkv
    idx = block_tables.clamp(min=0).long()
    L = idx.shape[1] * bs
    k = k_cache[idx].reshape(B, L, hkv, d)          # dense gather, bf16
    v = v_cache[idx].reshape(B, L, hkv, d)
    kt = k.permute(0, 2, 3, 1).float().contiguous()  # [B, Hkv, D, L]
    vf = v.permute(0, 2, 1, 3).float().contiguous()  # [B, Hkv, L, D]
    qf = q.float().reshape(B, hkv, g, d).contiguous()
    s = torch.matmul(qf, kt) * scale                 # [B, Hkv, G, L]
    live = torch.arange(L, device=q.device)[None, :] < context_lens[:, None].long()
    s = s.masked_fill(~live[:, None, None, :], float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = torch.matmul(p, vf).reshape(B, hq, d)
    return out.to(q.dtype), (k, v)


def gather_then_sdpa(q, k_cache, v_cache, block_tables, context_lens, scale):
    """The same prior art with PyTorch's fused attention: gather the pages to
    dense padded tensors, then ``scaled_dot_product_attention`` with a
    length mask and the query heads grouped over the kv heads (barellm
    README, feature list: pages gathered into dense tensors before PyTorch
    SDPA).  Attention runs in float32 (whichever backend PyTorch picks for a
    masked float32 call).  Returns out [B, Hq, D] in q's dtype."""
    import torch
    import torch.nn.functional as F
    B, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    idx = block_tables.clamp(min=0).long()
    L = idx.shape[1] * bs
    k = k_cache[idx].reshape(B, L, hkv, d).transpose(1, 2).float()   # [B, Hkv, L, D]
    v = v_cache[idx].reshape(B, L, hkv, d).transpose(1, 2).float()
    live = torch.arange(L, device=q.device)[None, :] < context_lens[:, None].long()
    out = F.scaled_dot_product_attention(q.float().reshape(B, hq, 1, d), k, v,
                                         attn_mask=live[:, None, None, :], scale=scale,
                                         enable_gqa=hq != hkv)
    return out.reshape(B, hq, d).to(q.dtype)


def stream_probe(torch, per_wg_bytes: int = 4 << 20) -> dict:
    """HBM streaming rates of plain reads (read_ceiling.hip rc_stream_probe):
    8, 64 and 256 workgroups, each streaming its own 4 MiB with 8 16-byte
    loads per lane in flight (8 waves: 64 KiB per workgroup; 16 waves: 128
    KiB), non-temporal and plain.  Workgroups are dealt to the 8 XCDs in
    turn, so 8 puts one reading CU on each XCD and 256 one on every CU.
    Every launch reads a region that no earlier launch of the probe read
    (the 2 GiB buffer is 8x the last-level cache; at 256 workgroups each
    launch reads 1 GiB); the median of the last 3 of 4 launches is reported."""
    import ctypes
    path = os.path.join(ROOT, "libreadceiling.so")
    if not os.path.exists(path):
        from paged_kv_cache_reshape_amd import build as _b
        _b.build_read_ceiling()
    lib = ctypes.CDLL(path)
    f = lib.rc_stream_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    total = 2 << 30
    buf = torch.randint(0, 1 << 30, (total // 4,), dtype=torch.int32, device=dev)
    sink = torch.zeros(2048, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    per_wg = per_wg_bytes // 16
    u = 8
    rows = []
    for nwg in (8, 64, 256):
        span = nwg * per_wg_bytes
        nregions = total // span
        k = 0
        for threads in (512, 1024):
            for nt in (1, 0):
                times = []
                for rep in range(4):
                    off = (k % nregions) * span
                    k += 1
                    assert off + span <= total
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record(stream)
                    st = f(buf.data_ptr() + off, per_wg, nwg, threads, u, nt, sink.data_ptr(),
                           stream.cuda_stream)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    if st != 0:
                        raise RuntimeError(f"rc_stream_probe: status {st}")
                    times.append(e0.elapsed_time(e1) * 1e3)
                t = float(np.median(times[1:]))
                rows.append({"workgroups": nwg, "waves": threads // 64,
                             "in_flight_kib": threads * u * 16 // 1024, "non_temporal": bool(nt),
                             "us": round(t, 1), "per_cu_gbs": round(per_wg_bytes / t / 1e3, 1),
                             "total_tbs": round(span / t / 1e6, 2)})
    return {"kind": "HBM streaming probe (read_ceiling.hip rc_stream_probe): each workgroup "
                    "streams its own 4 MiB, cold", "rows": rows}


def read_ceilings(torch, w, inp, kcs, vcs, tables, lens, stream, n: int):
    """Mean µs per launch of the pure-read kernels of ``read_ceiling.hip``
    (same bytes as the decode's K/V reads, no arithmetic) over n launches
    cycling the pool copies, HIP events on `stream`: the floor each access
    pattern puts under a decode.  None where they are not built for the
    workload (bfloat16 caches only) or the library is missing."""
    import ctypes
    path = os.path.join(ROOT, "libreadceiling.so")
    if w.dtype != "bf16" or not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    f = lib.rc_read_ceiling
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_void_p,
                  ctypes.c_void_p]
    ctx = inp["context_lens"].astype(np.int64)
    mb = tables.shape[1]
    blocks = int(np.minimum(-(-ctx // w.block_size), mb).sum())
    blk_bytes = w.block_size * w.num_kv_heads * w.head_dim * w.elt_bytes
    nbytes = 2 * blocks * blk_bytes
    sink = torch.zeros(2048, dtype=torch.int32, device=tables.device)
    R = len(kcs)

    def launch(mode, i):
        st = f(mode, kcs[i % R].data_ptr(), vcs[i % R].data_ptr(), tables.data_ptr(),
               lens.data_ptr(), w.num_seqs, mb, w.num_kv_heads, w.head_dim, w.block_size,
               nbytes, blocks, sink.data_ptr(), stream.cuda_stream)
        if st not in (0, -1):
            raise RuntimeError(f"rc_read_ceiling mode {mode}: HIP error {st}")
        return st == 0

    out = {"kind": "pure-read kernels (read_ceiling.hip): the decode's K/V bytes, no "
                   "arithmetic, 256 workgroups",
           "bytes": nbytes}
    for mode, name in ((0, "contiguous"), (1, "head_rows"), (2, "token_rows"),
                       (3, "head_interleaved")):
        if not launch(mode, 0):  # ranges longer than the kernel is built for
            out[name + "_us"] = None
            continue
        for i in range(1, 5):
            launch(mode, i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            launch(mode, i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        out[name + "_us"] = round(us, 3)
        out[name + "_gbs"] = round(nbytes / us / 1e3, 1)
    return out


def _one_thread():
    """Context that holds the BLAS / OpenMP pools to one thread."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1)


def _threads_used(cpu_s: float, wall_s: float) -> int:
    """Threads a timed CPU region kept busy: process CPU time over wall time."""
    return max(1, int(round(cpu_s / wall_s))) if wall_s > 0 else 1


def _oracle_decode_sample(inp: dict, budget_s: float):
    """The oracle's KV write, then its decode of the batch's sequences in
    order until budget_s has passed.  Returns (KV bytes, sequences, wall s,
    process CPU s)."""
    import oracle
    w = inp["workload"]
    B = w.num_seqs
    done_bytes = 0
    seqs_done = 0
    t0, c0 = time.perf_counter(), time.process_time()
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    b = 0
    while True:
        sel = [b % B]
        oracle.decode(inp["q"][sel], k, v, inp["block_tables"][sel],
                      inp["context_lens"][sel], inp["scale"], w.dtype)
        c = int(inp["context_lens"][b % B])
        done_bytes += (c * 2 * w.num_kv_heads * w.head_dim * w.elt_bytes
                       + 2 * w.num_q_heads * w.head_dim * w.elt_bytes)
        seqs_done += 1
        b += 1
        if time.perf_counter() - t0 >= budget_s and seqs_done >= min(B, 4):
            break
    return done_bytes, seqs_done, time.perf_counter() - t0, time.process_time() - c0


_POOL_STATE: dict = {}


def _pool_worker(args):
    """One worker of the spread oracle: decode sequences wid, wid + P, ... of
    the batch (cycling) until budget_s has passed, on one thread, over the KV
    caches the parent wrote before forking."""
    import oracle
    wid, nproc, budget_s = args
    inp, k, v = _POOL_STATE["inp"], _POOL_STATE["k"], _POOL_STATE["v"]
    w = inp["workload"]
    B = w.num_seqs
    done, seqs, b = 0, 0, wid
    t0 = time.perf_counter()
    with _one_thread():
        while True:
            sel = [b % B]
            oracle.decode(inp["q"][sel], k, v, inp["block_tables"][sel],
                          inp["context_lens"][sel], inp["scale"], w.dtype)
            c = int(inp["context_lens"][b % B])
            done += (c * 2 * w.num_kv_heads * w.head_dim * w.elt_bytes
                     + 2 * w.num_q_heads * w.head_dim * w.elt_bytes)
            seqs += 1
            b += nproc
            if time.perf_counter() - t0 >= budget_s:
                break
    return done, seqs


def _oracle_pool_sample(inp: dict, budget_s: float, nproc: int):
    """The oracle's KV write, then its decode spread over nproc forked worker
    processes for budget_s.  Returns (KV bytes, sequences, wall s)."""
    import multiprocessing as mp

    import oracle
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    _POOL_STATE.update(inp=inp, k=k, v=v)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(nproc) as pool:
        res = pool.map(_pool_worker, [(i, nproc, budget_s) for i in range(nproc)])
    dt = time.perf_counter() - t0
    _POOL_STATE.clear()
    return sum(r[0] for r in res), sum(r[1] for r in res), dt


def cpu_baseline(inp: dict, budget_s: float) -> dict:
    """Time the float64 oracle's write + decode on a bounded sample of the
    batch: spread over the host's cores (one worker process each, at most
    CPU_POOL_MAX, every worker on one thread: the headline figure), and on one
    thread alone.  `cores` is the number of worker processes used,
    `host_cores` the cores this process may run on."""
    host = len(os.sched_getaffinity(0))
    nproc = max(1, min(host, CPU_POOL_MAX))
    nb, ns, dt = _oracle_pool_sample(inp, budget_s, nproc)
    with _one_thread():
        nb1, ns1, dt1, _ = _oracle_decode_sample(inp, budget_s / 3)
    return {"value": round(nb / dt / 1e9, 4), "unit": "GB/s",
            "cores": nproc, "host_cores": host, "kind": "oracle",
            "sample": (f"float64 numpy oracle: one full-pool KV write, then decode of "
                       f"{ns} sequences of this batch (cycling) over {nproc} worker "
                       f"processes of one thread each ({dt:.1f} s wall, "
                       f"{nb / 1e6:.1f} MB of KV rows)"),
            "one_thread": {"value": round(nb1 / dt1 / 1e9, 4), "unit": "GB/s",
                           "sample": f"same on one thread: {ns1} sequences in order "
                                     f"({dt1:.1f} s)"}}


def cpu_baseline_child(workload: str, budget_s: float) -> dict:
    """cpu_baseline in a child process started before this process touches
    the GPU (its worker pool forks from a process that never did)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                        "--workload", workload, "--cpu-seconds", str(budget_s)],
                       capture_output=True, text=True, check=True)
    return json.loads(r.stdout.strip().splitlines()[-1])


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def prefill_flops(inp: dict) -> int:
    """Attention flops of one prefill launch: each new row at position p
    does q.k and p.v over p + 1 keys, 2 * D flops each, for every query head."""
    w = inp["workload"]
    ctx, start = inp["context_lens"].astype(np.int64), inp["query_start"].astype(np.int64)
    n = start[1:] - start[:-1]
    # sum over rows of (p + 1) with p = ctx - n + i, i < n
    keys = (n * (ctx - n) + n * (n + 1) // 2).sum()
    return int(4 * w.num_q_heads * w.head_dim * keys)


def _oracle_prefill_sample(inp: dict, budget_s: float):
    """The oracle's prefill of the batch's new tokens in order, one row at a
    time, until budget_s has passed.  Returns (flops, rows, wall s, CPU s)."""
    import oracle
    w = inp["workload"]
    ctx, start = inp["context_lens"], inp["query_start"]
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    flops, rows = 0, 0
    t0, c0 = time.perf_counter(), time.process_time()
    for b in range(len(ctx)):
        lo, hi = int(start[b]), int(start[b + 1])
        for i in range(hi - lo):
            one = np.array([0, 1], dtype=np.int32)
            pos = int(ctx[b]) - (hi - lo) + i
            oracle.prefill(inp["q"][lo + i:lo + i + 1], k, v, inp["block_tables"][b:b + 1],
                           np.array([pos + 1], dtype=np.int32), one, inp["scale"], w.dtype)
            flops += 4 * w.num_q_heads * w.head_dim * (pos + 1)
            rows += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    return flops, rows, time.perf_counter() - t0, time.process_time() - c0


def prefill_cpu_baseline(inp: dict, budget_s: float) -> dict:
    """Time the float64 oracle's prefill on the batch's first new tokens, with
    the thread pools as they are and held to one thread; `cores` as in
    cpu_baseline."""
    fl, rows, dt, cpu = _oracle_prefill_sample(inp, budget_s)
    with _one_thread():
        fl1, rows1, dt1, _ = _oracle_prefill_sample(inp, budget_s / 3)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": _threads_used(cpu, dt), "kind": "oracle",
            "sample": f"float64 numpy oracle prefill, the first {rows} new tokens of the "
                      f"batch in order ({dt:.1f} s)",
            "one_thread": {"value": round(fl1 / dt1 / 1e12, 6), "unit": "TFLOP/s",
                           "sample": f"same, the first {rows1} new tokens with the thread "
                                     f"pools held to one thread ({dt1:.1f} s)"}}


def run_prefill(args, torch, pa, cpu_base) -> int:
    """Prefill step: write every new token's K/V rows, then causal prefill
    attention over the paged cache.  value = attention TFLOP/s of the step."""
    w = synth.PREFILL_WORKLOADS[args.workload]
    inp = synth.make_prefill_inputs(w)
    dev = torch.device("cuda:0")

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    pool_bytes = 2 * inp["k_cache"].nbytes
    R = args.replicas or min(64, max(1, math.ceil(1.25 * 2**30 / pool_bytes)))
    kcs = [up(inp["k_cache"])]
    vcs = [up(inp["v_cache"])]
    kcs += [kcs[0].clone() for _ in range(R - 1)]
    vcs += [vcs[0].clone() for _ in range(R - 1)]
    q, key, value = up(inp["q"]), up(inp["key"]), up(inp["value"])
    tables, lens = up(inp["block_tables"]), up(inp["context_lens"])
    qstart, slots = up(inp["query_start"]), up(inp["slot_mapping"])
    scale = float(inp["scale"])
    out = torch.empty_like(q)
    mq = int(inp["max_query_len"])
    stream = torch.cuda.current_stream(dev)

    def write(i):
        pa.reshape_and_cache(key, value, kcs[i % R], vcs[i % R], slots)

    def attn(i):
        pa.paged_attention_prefill(q, kcs[i % R], vcs[i % R], tables, lens, qstart, scale,
                                   max_query_len=mq, out=out)

    def step(i):
        write(i)
        attn(i)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    steps = min(args.steps, 200)
    warm = min(args.warmup, 20)
    for i in range(warm):
        step(i)
    ms_step = timed(step, steps)
    ms_attn = timed(attn, steps)
    ms_write = timed(write, steps)
    flops = prefill_flops(inp)
    T = int(inp["query_start"][-1])
    achieved = flops / (ms_attn / 1e3) / 1e12
    res = {
        "metric": "prefill attention TFLOP/s (causal, paged cache)",
        "value": round(flops / (ms_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
                         f"D={w.head_dim} block_size={w.block_size} ctx {w.ctx} "
                         f"new tokens {w.query} {w.dtype}"),
            "new_tokens": T,
            "sum_ctx": int(inp["context_lens"].sum()),
            "kv_pool_replicas": R,
            "step": "reshape_and_cache (all new tokens) + paged_attention_prefill",
        },
        "tokens_per_s": round(T / (ms_step / 1e3), 1),
        "prefill_us_mean": round(ms_attn * 1e3, 3),
        "write_us_mean": round(ms_write * 1e3, 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": "prefill_mfma_kernel",
            "flops_per_launch": flops,
        },
    }
    if cpu_base is not None:
        res["cpu_baseline"] = cpu_base
    print(json.dumps(res), flush=True)
    return 0


TIMELINE_LIB = os.path.join(ROOT, "paged_kv_cache_reshape_amd", "_build_timeline",
                            "libpagedattn_timeline.so")


def timeline_library() -> str:
    """The measurement build of the library (PA_TIMELINE: the stream kernel's
    waves stamp the GPU's constant clock), built beside the normal one."""
    if not os.path.exists(TIMELINE_LIB):
        from paged_kv_cache_reshape_amd import build as _b
        _b.build(defines=["PA_TIMELINE=1"], out=TIMELINE_LIB)
    return TIMELINE_LIB


def timeline_summary(lib, reader: str = "pa_debug_timeline") -> dict:
    """Per-wave clock stamps of the last stream-kernel launch since the last
    read (the reader clears the records), as offsets
    from its first wave's start (us): when each wave had requested its first
    block (prologue), ended its range (stream) and was done (after its merge,
    if it merged)."""
    import ctypes
    words = 16384 * 8
    buf = (ctypes.c_ulonglong * words)()
    khz = ctypes.c_int32()
    fn = getattr(lib, reader)
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    n = fn(buf, words, ctypes.byref(khz))
    if n <= 0 or khz.value <= 0:
        raise RuntimeError("pa_debug_timeline failed")
    return timeline_stats(np.frombuffer(buf, dtype=np.uint64).reshape(-1, 8).astype(np.int64),
                          khz.value)


def timeline_stats(rec: np.ndarray, clock_khz: int) -> dict:
    """Summary of per-wave records [t_start, t_prologue, t_stream, t_done,
    hw ids, pieces merged (0: not a merger), t_lengths, t_range], clock ticks
    at clock_khz (t_lengths / t_range: 0 where not recorded)."""
    tick_us = 1000.0 / clock_khz
    # The reader clears the records, and every launch of the same grid
    # rewrites its waves' records: only the last launch's waves hold stamps,
    # and those that stream (not the copy workgroups) hold all four.
    r = rec[(rec[:, 0] > 0) & (rec[:, 1] >= rec[:, 0]) & (rec[:, 2] >= rec[:, 1])
            & (rec[:, 3] >= rec[:, 2])]
    if len(r) == 0:
        raise RuntimeError("no stream-kernel wave recorded a timeline")
    base = r[:, 0].min()
    us = (r[:, :4] - base) * tick_us
    merger = r[:, 5] > 0
    xcc = (r[:, 4] >> 32) & 0xF
    q = lambda a, p: round(float(np.percentile(a, p)), 2)
    crit = int(np.argmax(us[:, 3]))
    # Compute unit of each wave: XCC, shader engine, shader array and CU of
    # HW_ID; waves per CU tell whether some CUs host more workgroups.
    hw = r[:, 4]
    cu_key = (((hw >> 32) & 0xF) << 8) | (((hw >> 13) & 0x7) << 5) | (((hw >> 12) & 1) << 4) \
        | ((hw >> 8) & 0xF)
    _, per_cu = np.unique(cu_key, return_counts=True)
    waves_per_cu = {int(k): int(v) for k, v in zip(*np.unique(per_cu, return_counts=True))}
    cu_of = {int(k): i for i, k in enumerate(np.unique(cu_key))}
    cu_end = np.zeros(len(cu_of))
    for k, e in zip(cu_key, us[:, 2]):
        cu_end[cu_of[int(k)]] = max(cu_end[cu_of[int(k)]], e)
    return {
        "kind": "per-wave GPU constant-clock stamps, latest launch of the stream kernel "
                "(measurement build PA_TIMELINE)",
        "clock_khz": int(clock_khz),
        "waves": int(len(r)),
        "mergers": int(merger.sum()),
        "start_us": {"max": q(us[:, 0], 100)},
        "lengths_end_us": ({"median": q((r[:, 6] - base) * tick_us, 50),
                            "max": q((r[:, 6] - base) * tick_us, 100)}
                           if r.shape[1] > 6 and (r[:, 6] > 0).all() else None),
        "range_end_us": ({"median": q((r[:, 7] - base) * tick_us, 50),
                          "max": q((r[:, 7] - base) * tick_us, 100)}
                         if r.shape[1] > 7 and (r[:, 7] > 0).all() else None),
        "prologue_end_us": {"median": q(us[:, 1], 50), "p90": q(us[:, 1], 90),
                            "max": q(us[:, 1], 100)},
        "stream_end_us": {"min": q(us[:, 2], 0), "median": q(us[:, 2], 50),
                          "p90": q(us[:, 2], 90), "max": q(us[:, 2], 100)},
        "stream_end_us_per_xcd_max": [q(us[xcc == x, 2], 100) for x in range(8)
                                      if (xcc == x).any()],
        "merge_us": ({"median": q(us[merger, 3] - us[merger, 2], 50),
                      "max": q(us[merger, 3] - us[merger, 2], 100)} if merger.any() else None),
        "done_us_max": q(us[:, 3], 100),
        "last_wave": {"stream_end_us": round(float(us[crit, 2]), 2),
                      "done_us": round(float(us[crit, 3]), 2), "merger": bool(merger[crit])},
        "last_stream_end_to_done_us": round(float(us[:, 3].max() - us[:, 2].max()), 2),
        "compute_units": len(cu_of),
        "cus_by_waves_hosted": waves_per_cu,
        "cu_stream_end_us": {"min": q(cu_end, 0), "median": q(cu_end, 50), "max": q(cu_end, 100)},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # Untimed steps before the timed ones.  The GPU's clocks take longer than
    # 50 steps to settle after the idle CPU-baseline phase: measured on
    # MI355X, 50 warm-up steps left the timed Qwen3 steps at 33.0 us and the
    # Llama-3.2 ones at 52.0 us, against 32.7 and 50.7 us after 3000 (the
    # decode loops timed later in the same run read the same either way).
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--workload", default="qwen3_0p6b",
                    choices=sorted(synth.WORKLOADS) + sorted(synth.PREFILL_WORKLOADS),
                    help="a decode batch, or a prefill batch (prefill_*, chunked_*)")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="tokens per partition; -1 = the workload's, 0 = library choice")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for 1.25 GiB")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--no-prior-art", action="store_true",
                    help="skip timing the gather-then-attention PyTorch baseline")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="print the CPU baseline of the workload as JSON and exit (no GPU)")
    ap.add_argument("--step-only", action="store_true",
                    help="time the steps only (no separate decode, write or graph timing), "
                         "so that every decode-kernel launch is a fused step: for counter runs")
    ap.add_argument("--timeline", action="store_true",
                    help="run the steps on the measurement build of the library (PA_TIMELINE) "
                         "and add the per-wave timeline of the last launch (balanced schedule)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="print the HBM streaming rates of 8, 64 and 256 reading workgroups "
                         "(read_ceiling.hip rc_stream_probe) as JSON and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(no sharding, no collectives); run with --gpus 1.", file=sys.stderr)
        return 2

    if args.cpu_baseline_only:
        if args.workload in synth.PREFILL_WORKLOADS:
            base = prefill_cpu_baseline(synth.make_prefill_inputs(
                synth.PREFILL_WORKLOADS[args.workload]), args.cpu_seconds)
        else:
            base = cpu_baseline(synth.make_inputs(synth.WORKLOADS[args.workload]),
                                args.cpu_seconds)
        print(json.dumps(base), flush=True)
        return 0
    if args.stream_probe:
        import torch
        print(json.dumps(stream_probe(torch)), flush=True)
        return 0
    # The CPU baseline runs first, in a child process, before anything here
    # touches the GPU.
    cpu_base = None if args.no_cpu_baseline else cpu_baseline_child(args.workload,
                                                                    args.cpu_seconds)

    import torch
    import paged_kv_cache_reshape_amd as pa
    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_reshape_amd import build as _b
        _b.build()
    if args.timeline:
        args.step_only = True
        pa.LIB_PATH = timeline_library()
    pa.load_library()
    if args.workload in synth.PREFILL_WORKLOADS:
        return run_prefill(args, torch, pa, cpu_base)

    w = synth.WORKLOADS[args.workload]
    ps = w.partition_size if args.partition_size < 0 else args.partition_size
    inp = synth.make_inputs(w)
    nbytes = algorithmic_bytes(inp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        if w.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    pool_bytes = 2 * inp["k_cache"].nbytes
    # Enough pool copies that one pass over them (1.25 GiB) cannot sit in the
    # caches; at most 64 (tiny pools are launch-bound anyway).
    R = args.replicas or min(64, max(1, math.ceil(1.25 * 2**30 / pool_bytes)))
    kc0, vc0 = up(inp["k_cache"]), up(inp["v_cache"])
    kcs = [kc0] + [kc0.clone() for _ in range(R - 1)]
    vcs = [vc0] + [vc0.clone() for _ in range(R - 1)]
    q, key, value = up(inp["q"]), up(inp["key"]), up(inp["value"])
    tables = torch.from_numpy(inp["block_tables"]).to(dev)
    lens = torch.from_numpy(inp["context_lens"]).to(dev)
    slots = torch.from_numpy(inp["slot_mapping"]).to(dev)
    scale = float(inp["scale"])
    out = torch.empty_like(q)
    hq, hkv, d, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    ws_bytes = pa.decode_workspace_bytes(w.num_seqs, hq, hkv, d, tables.shape[1], bs, ps)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    counters = torch.zeros(w.num_seqs * hkv, dtype=torch.int32, device=dev)
    part = pa.decode_partition_size(w.num_seqs, hq, hkv, d, tables.shape[1], bs, ps)

    stream = torch.cuda.current_stream(dev)

    def write(i):
        r = i % R
        pa.reshape_and_cache(key, value, kcs[r], vcs[r], slots)

    def decode(i):
        r = i % R
        pa.paged_attention_decode(q, kcs[r], vcs[r], tables, lens, scale,
                                  partition_size=ps, out=out, workspace=ws,
                                  counters=counters)

    def unfused(i):
        write(i)
        decode(i)

    def step(i):
        r = i % R
        pa.decode_step(q, key, value, kcs[r], vcs[r], tables, lens, scale,
                       partition_size=ps, out=out, workspace=ws, counters=counters)

    def timed(fn, n, first):
        """Mean ms per call of n back-to-back calls, HIP events on `stream`."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(first + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    if args.step_only:
        cal = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        cal.clone()
        torch.cuda.synchronize()
        del cal
    for i in range(args.warmup):
        step(i)
    # The timed region: K whole steps.
    ms_step = timed(step, args.steps, args.warmup)
    # Per-kernel means over K back-to-back launches of each kernel (no events
    # between launches, so the figures compare with a kernel trace).
    k_mean_s = w_mean_s = unfused_ms = warm_s = None
    loops_us = []
    if not args.step_only:
        k_mean_s = timed(decode, args.steps, args.warmup + args.steps) / 1e3
        w_mean_s = timed(write, args.steps, args.warmup) / 1e3
        unfused_ms = timed(unfused, args.steps, args.warmup)
        # Spread: five more loops of decode launches, each timed on its own.
        n_loop = max(20, args.steps // 5)
        loops_us = [timed(decode, n_loop, j * n_loop) * 1e3 for j in range(5)]

        # Warm single pool: every launch reads the same pool copy, which the
        # 256 MB last-level cache can hold when the pool is smaller than it.
        def decode_one_pool(i):
            pa.paged_attention_decode(q, kc0, vc0, tables, lens, scale, partition_size=ps,
                                      out=out, workspace=ws, counters=counters)
        for i in range(3):
            decode_one_pool(i)
        warm_s = timed(decode_one_pool, args.steps, 0) / 1e3

    # The same steps replayed from a HIP graph (one graph holds one step per
    # pool copy); buffers were all allocated above, so capture allocates nothing.
    graph_us = None
    if not args.no_graph and not args.step_only:
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(R):
                step(i)
        reps = max(1, args.steps // R)
        graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / (reps * R)
        del graph

    prior = None
    if not args.no_prior_art and not args.step_only:
        n_pa = 20
        for i in range(3):
            gather_then_attention(q, kcs[i % R], vcs[i % R], tables, lens, scale)
        pa_ms = timed(lambda i: gather_then_attention(q, kcs[i % R], vcs[i % R], tables,
                                                      lens, scale), n_pa, 0)
        for i in range(3):
            gather_then_sdpa(q, kcs[i % R], vcs[i % R], tables, lens, scale)
        sd_ms = timed(lambda i: gather_then_sdpa(q, kcs[i % R], vcs[i % R], tables, lens,
                                                 scale), n_pa, 0)
        idx = tables.clamp(min=0).long()
        ga_ms = timed(lambda i: (kcs[i % R][idx], vcs[i % R][idx]), n_pa, 0)
        prior = {
            "kind": "PyTorch: gather pages to dense padded bf16, then attention in fp32",
            "us_per_decode": round(pa_ms * 1e3, 3),
            "matmul_softmax_us": round(pa_ms * 1e3, 3),
            "sdpa_us": round(sd_ms * 1e3, 3),
            "dense_gather_us": round(ga_ms * 1e3, 3),
            "decode_speedup": round(pa_ms / (k_mean_s * 1e3), 2),
            "decode_speedup_vs_sdpa": round(sd_ms / (k_mean_s * 1e3), 2),
        }

    timeline = None
    if args.timeline:
        if part != 0:
            raise SystemExit("--timeline covers the balanced schedule's kernels only")
        reader = ("pa_debug_timeline_mfma" if decode_kernel_name(w, part)
                  == "decode_stream_mfma_kernel" else "pa_debug_timeline")
        timeline_summary(pa.load_library(), reader)  # clears the records
        # Back-to-back steps as in the timed region; each launch rewrites its
        # waves' records, so the read holds the last one.
        for i in range(args.steps):
            step(args.warmup + args.steps + i)
        timeline = timeline_summary(pa.load_library(), reader)

    ceilings = None
    if not args.step_only:
        ceilings = read_ceilings(torch, w, inp, kcs, vcs, tables, lens, stream, args.steps)

    achieved = nbytes["step"] / (ms_step / 1e3) / 1e9
    traffic = None
    rec = traffic_record(w.name)
    if (rec and rec.get("workload") == w.name and rec.get("partition_size") == part
            and rec.get("launch") == "fused step"):
        traffic = rec.get("hbm_bytes_per_launch")
    res = {
        "metric": METRIC,
        "value": round(nbytes["step"] / (ms_step / 1e3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: B={w.num_seqs} Hq={hq} Hkv={hkv} D={d} "
                         f"block_size={bs} ctx {w.ctx} {w.dtype}"),
            "sum_ctx": int(inp["context_lens"].sum()),
            "partition_size": part,
            "kv_pool_replicas": R,
            "step": "decode_step: the KV write of each new token fused into the decode launch",
        },
        "us_per_step": round(ms_step * 1e3, 3),
        "tokens_per_s": round(w.num_seqs / (ms_step / 1e3), 1),
        "unfused_us_per_step": None if unfused_ms is None else round(unfused_ms * 1e3, 3),
        "decode_us_mean": None if k_mean_s is None else round(k_mean_s * 1e6, 3),
        "write_us_mean": None if w_mean_s is None else round(w_mean_s * 1e6, 3),
        "decode_kv_gbs": None if k_mean_s is None else round(nbytes["kv"] / k_mean_s / 1e9, 3),
        "decode_us_loops": [round(x, 3) for x in loops_us],
        "decode_us_median": round(float(np.median(loops_us)), 3) if loops_us else None,
        "mall_resident": None if warm_s is None else {
            "decode_us_mean": round(warm_s * 1e6, 3),
            "decode_gbs": round(nbytes["decode"] / warm_s / 1e9, 3),
            "pool_bytes": int(pool_bytes),
            "note": "one pool copy read by every launch (warm caches), not HBM-bound "
                    "when the pool fits the 256 MB last-level cache",
        },
        "cache_line_efficiency": (None if not traffic
                                  else round(nbytes["step"] / traffic, 4)),
        "graph_us_per_step": None if graph_us is None else round(graph_us, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": decode_kernel_name(w, part) + " (KV write fused)",
            "bytes_per_launch": nbytes["step"],
        },
    }
    if ceilings is not None:
        res["read_ceiling"] = ceilings
    if timeline is not None:
        res["timeline"] = timeline
    if prior is not None:
        res["prior_art"] = prior
    if cpu_base is not None:
        res["cpu_baseline"] = cpu_base
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
