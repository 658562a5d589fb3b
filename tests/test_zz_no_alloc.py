"""The decode step that allocates nothing (pa_decode_step_noalloc) against the
decode step with a caller-owned workspace (pa_decode_step), through the C ABI.

Both run the same kernels, so the outputs and the written caches must agree
bit for bit; the output is also checked against the float64 oracle at the
tolerance of every decode test.  Calls follow one another on one GPU, each
with a smaller batch than the one before, so every call finds the previous
call's partials and counters in the shared device buffer.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import paged_kv_cache_reshape_amd as pa
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def subset(inp, n):
    """The first n sequences of a generated batch (same pool, same caches)."""
    out = dict(inp)
    for k in ("q", "key", "value", "block_tables", "context_lens", "slot_mapping"):
        out[k] = inp[k][:n].copy()
    return out


def oracle_step(inp):
    w = inp["workload"]
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    return oracle.decode(inp["q"], k, v, inp["block_tables"], inp["context_lens"],
                         inp["scale"], w.dtype), (k, v)


def both_steps(inp, ps):
    """pa_decode_step and pa_decode_step_noalloc on two uploads of `inp`."""
    d1, d2 = G.upload(inp), G.upload(inp)
    want = pa.decode_step(d1["q"], d1["key"], d1["value"], d1["k_cache"], d1["v_cache"],
                          d1["block_tables"], d1["context_lens"], d1["scale"],
                          partition_size=ps)
    out = torch.full_like(d2["q"], float("nan"))
    got = pa.decode_step_noalloc(d2["q"], d2["key"], d2["value"], d2["k_cache"],
                                 d2["v_cache"], d2["block_tables"], d2["context_lens"],
                                 d2["scale"], out, partition_size=ps)
    assert got is out
    torch.cuda.synchronize()
    return d1, want, d2, got


def check(inp, ps, what):
    say("noalloc", what, "partition", ps)
    d1, want, d2, got = both_steps(inp, ps)
    assert np.array_equal(G.host_storage(got), G.host_storage(want)), what
    for c in ("k_cache", "v_cache"):
        assert torch.equal(d1[c], d2[c]), (what, c)
    ref, (k_ref, v_ref) = oracle_step(inp)
    G.assert_close(G.host_f64(got), ref, inp["workload"].dtype, what)
    assert np.array_equal(G.host_storage(d2["k_cache"]), k_ref), what
    assert np.array_equal(G.host_storage(d2["v_cache"]), v_ref), what


def test_noalloc_matches_workspace_step_on_shrinking_batches():
    """Qwen3-shaped batch (balanced schedule, in-launch merge with arrival
    counters), then its first 11 sequences, then a tiny float32 batch."""
    qwen = G.cached_inputs("qwen3_0p6b")
    check(qwen, 0, "qwen3_0p6b, 32 sequences")
    check(subset(qwen, 11), 0, "qwen3_0p6b, 11 sequences")
    check(G.cached_inputs("tiny_f32"), 0, "tiny_f32")


def test_noalloc_fixed_schedule_both_merge_paths():
    """Llama-3.2-shaped batch on the fixed schedule: 1024-token partitions
    merged in the launch (counters), then 256-token partitions (16 per
    sequence) merged by the second kernel with 8 MiB of partials, then half
    the batch at 1024 again."""
    inp = G.cached_inputs("llama32_1b")
    check(inp, 1024, "llama32_1b, in-launch merge")
    check(inp, 256, "llama32_1b, separate merge")
    check(subset(inp, 32), 1024, "llama32_1b, 32 sequences")


def test_noalloc_refuses_sizes_beyond_its_buffer():
    """More workspace than the static buffer holds: an error before any
    launch, and the buffer still serves the next call."""
    w = synth.Workload("noalloc_big", 8, 32, 8, 128, 16, "bf16", ("uniform", 100, 900),
                       seed=5)
    inp = synth.make_inputs(w)
    d = G.upload(inp)
    wide = torch.zeros((8, 4096), dtype=torch.int32, device="cuda")
    wide[:, : d["block_tables"].shape[1]] = d["block_tables"]
    out = torch.empty_like(d["q"])
    with pytest.raises(pa.PagedAttnError, match="noalloc"):
        pa.decode_step_noalloc(d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"],
                               wide, d["context_lens"], d["scale"], out, partition_size=512)
    check(inp, 0, "after a refused call")
