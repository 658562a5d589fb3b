"""Seeded sweeps of small random shapes: the HIP path against the float64
oracle, through the C ABI, on combinations the fixed shapes do not reach.

Each case draws, from its own seed, the element type, head size, block size,
query heads per kv head, kv heads, batch size, the spread of context lengths
(empty sequences included) and the partition size (or the library's choice),
and checks both the write + decode calls and the fused step against the
oracle, and the two against each other bit for bit; for the prefill, whole
prompts or chunks and the key-halves form.  The bar is the one of the other
parity tests (tests/_gpu.py): bf16 2e-3 + 1e-2|y| elementwise, max abs 2e-3
below |y| = 0.5, max rel 1e-2 above |y| = 0.2; f32 1e-5 + 1e-5|y|.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_reshape_amd as pa
import synth
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def decode_case(seed: int):
    rng = np.random.default_rng(10_000 + seed)
    dtype = str(rng.choice(["bf16", "f32"]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    grp = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hkv = int(rng.choice([1, 2, 4])) if grp <= 16 else 1
    B = int(rng.integers(1, 13))
    top = int(rng.choice([16, 100, 700, 2100]))
    w = synth.Workload(f"rand{seed}", B, grp * hkv, hkv, D, bs, dtype, ("uniform", 0, top),
                       seed=20_000 + seed)
    blocks = w.max_blocks_per_seq
    part = 0 if rng.random() < 0.4 else bs * int(rng.integers(1, min(blocks, 128) + 1))
    valu = dtype == "bf16" and grp >= 8 and rng.random() < 0.3
    return w, part, valu


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_shapes(seed, monkeypatch):
    w, part, valu = decode_case(seed)
    if valu:
        G.setopt(monkeypatch, "PAGEDATTN_DECODE_KERNEL", "valu")
    inp = synth.make_inputs(w)
    ctx = inp["context_lens"].copy()
    ctx[::5] = 0 if seed % 2 else ctx[::5]  # empty sequences in every other case
    inp = synth.make_inputs(w, context_lens=ctx)
    say("decode", w, "partition", part, "vector-ALU forced" if valu else "")
    d = G.upload(inp)
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    out = pa.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                    d["context_lens"], d["scale"], partition_size=part)
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    ref = oracle.decode(inp["q"], k, v, inp["block_tables"], inp["context_lens"],
                        inp["scale"], w.dtype)
    G.assert_close(G.host_f64(out), ref, w.dtype, f"random decode {seed}")
    # The fused step on fresh caches: the same bits, output and caches.
    d2 = G.upload(inp)
    out2 = pa.decode_step(d2["q"], d2["key"], d2["value"], d2["k_cache"], d2["v_cache"],
                          d2["block_tables"], d2["context_lens"], d2["scale"],
                          partition_size=part)
    assert np.array_equal(G.host_storage(out2), G.host_storage(out))
    assert torch.equal(d2["k_cache"], d["k_cache"]) and torch.equal(d2["v_cache"], d["v_cache"])
    G.assert_close(G.host_f64(out2), ref, w.dtype, f"random fused step {seed}")


def prefill_case(seed: int):
    rng = np.random.default_rng(30_000 + seed)
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    grp = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hkv = int(rng.choice([1, 2])) if grp <= 16 else 1
    B = int(rng.integers(1, 7))
    top = int(rng.choice([40, 300, 900]))
    query = ("full",) if rng.random() < 0.5 else ("uniform", 1, top)
    w = synth.Workload(f"rpf{seed}", B, grp * hkv, hkv, D, bs, "bf16", ("uniform", 1, top),
                       seed=40_000 + seed, query=query)
    return w, str(rng.choice(["1", "2"]))


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_shapes(seed, monkeypatch):
    w, ks = prefill_case(seed)
    G.setopt(monkeypatch, "PAGEDATTN_PREFILL_KSPLIT", ks)
    inp = synth.make_prefill_inputs(w)
    say("prefill", w, "key halves", ks)
    d = G.upload(inp)
    qstart = torch.from_numpy(inp["query_start"]).cuda()
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    out = pa.paged_attention_prefill(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                     d["context_lens"], qstart, d["scale"])
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    ref = oracle.prefill(inp["q"], k, v, inp["block_tables"], inp["context_lens"],
                         inp["query_start"], inp["scale"], "bf16")
    G.assert_close(G.host_f64(out), ref, "bf16", f"random prefill {seed}")
