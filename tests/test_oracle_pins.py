"""The CPU oracle against facts that do not come from the oracle (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests import _pins as P

W1 = synth.WORKLOADS["tiny_f32"]
SMALL = {
    "tiny_f32": W1,
    "gqa4_bf16": synth.Workload("gqa4_bf16", 6, 8, 2, 32, 16, "bf16",
                                ("uniform", 1, 100), num_blocks=48,
                                seed=21),
    "mqa_bf16_bs32": synth.Workload("mqa_bf16_bs32", 5, 4, 1, 16, 32, "bf16",
                                    ("uniform", 1, 90), sigma=0.5,
                                    num_blocks=24, seed=22),
    "mha_f32": synth.Workload("mha_f32", 3, 3, 3, 8, 16, "f32",
                              ("uniform", 2, 50), num_blocks=16,
                              seed=23),
}


def _ok(res):
    ok, detail = res
    assert ok, detail


# ------------------------------------------------------------ generator
def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    x[:6] = [0.0, -0.0, 1.0, 3.3895314e38, 1e-40, -2.5]
    got = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_generator_is_deterministic_and_seeded():
    a = synth.make_inputs(SMALL["gqa4_bf16"])
    b = synth.make_inputs(SMALL["gqa4_bf16"])
    c = synth.make_inputs(SMALL["gqa4_bf16"], seed=99)
    for key in ("context_lens", "block_tables", "k_cache", "v_cache", "q", "key",
                "value", "slot_mapping"):
        assert np.array_equal(a[key], b[key]), key
    assert not np.array_equal(a["k_cache"], c["k_cache"])


def test_generator_layout_facts():
    inp = synth.make_inputs(W1)
    assert list(inp["context_lens"]) == [1, 17, 33, 64]
    assert inp["k_cache"].shape == (32, 16, 2, 64)
    t = inp["block_tables"]
    used = t[t >= 0]
    assert len(np.unique(used)) == used.size == 1 + 2 + 3 + 4
    # the new token sits at position ctx-1: first slot of a block for 1, 17, 33
    offs = inp["slot_mapping"] % 16
    assert list(offs) == [0, 0, 0, 15]


def test_pool_rule():
    w = synth.WORKLOADS["qwen3_0p6b"]
    ctx = synth.draw_context_lens(w, np.random.default_rng(w.seed))
    nb = synth.pool_blocks(w, ctx)
    assert nb == max(int(np.ceil(1.25 * ctx.sum() / 16)),
                     int(sum(-(-c // 16) for c in ctx)))
    assert ctx.min() >= 128 and ctx.max() <= 2048


def test_widen_matches_torch_bf16():
    rng = np.random.default_rng(1)
    bits = synth.f32_to_bf16_bits(rng.standard_normal(5000).astype(np.float32))
    assert np.array_equal(oracle.widen(bits, "bf16"), P.widen_ref(bits, "bf16"))


# ------------------------------------------------------------ pins

def _golden_rows(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    rows = [line.split() for line in open(path) if line.strip() and not line.startswith("#")]
    return [tuple(int(v) for v in r) for r in rows]


def test_golden_tiny_newest_token():
    """The tiny batch's newest tokens, worked by hand from the paged-cache
    definition (tests/golden/tiny_newest_token.txt): the generator's slots, the
    oracle's write and the oracle's gather all put each new row there."""
    rows = _golden_rows("tiny_newest_token.txt")
    x = synth.make_inputs(W1)
    bs = W1.block_size
    assert [r[0] for r in rows] == [int(c) for c in x["context_lens"]]
    k2, v2 = oracle.reshape_and_cache(x["key"], x["value"], x["k_cache"], x["v_cache"],
                                      x["slot_mapping"])
    kd = oracle.gather_kv(k2, x["block_tables"], x["context_lens"])
    vd = oracle.gather_kv(v2, x["block_tables"], x["context_lens"])
    kd0 = oracle.gather_kv(x["k_cache"], x["block_tables"], x["context_lens"])
    for b, (ctx, pos, lblk, off, used) in enumerate(rows):
        table = x["block_tables"][b]
        assert int((table >= 0).sum()) == used
        assert int(x["slot_mapping"][b]) == int(table[lblk]) * bs + off
        assert np.array_equal(kd[b, pos].view(np.uint8), x["key"][b].view(np.uint8))
        assert np.array_equal(vd[b, pos].view(np.uint8), x["value"][b].view(np.uint8))
        # every earlier row of the sequence is untouched by the write
        assert np.array_equal(kd[b, :pos].view(np.uint8), kd0[b, :pos].view(np.uint8))

@pytest.mark.parametrize("name", list(SMALL))
def test_p1_write_slots(name):
    inp = synth.make_inputs(SMALL[name])
    inp["slot_mapping"][1] = -1  # a padding row writes nothing
    _ok(P.pin_write_slots(oracle.reshape_and_cache, inp))


@pytest.mark.parametrize("name", list(SMALL))
def test_p2_gather(name):
    _ok(P.pin_gather_chunks(oracle.gather_kv, synth.make_inputs(SMALL[name])))


@pytest.mark.parametrize("name", list(SMALL))
def test_p3_single_token(name):
    _ok(P.pin_single_token(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


@pytest.mark.parametrize("name", ["tiny_f32", "gqa4_bf16"])
def test_p4_onehot(name):
    _ok(P.pin_onehot(oracle.decode, SMALL[name]))


@pytest.mark.parametrize("name", list(SMALL))
def test_p5_block_permutation(name):
    _ok(P.pin_block_permutation(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


@pytest.mark.parametrize("name", ["tiny_f32", "gqa4_bf16", "mqa_bf16_bs32"])
def test_p6_gqa_equals_mha(name):
    _ok(P.pin_gqa_equals_mha(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


@pytest.mark.parametrize("name,ps", [("tiny_f32", 16), ("tiny_f32", 32),
                                     ("gqa4_bf16", 16), ("mqa_bf16_bs32", 32)])
def test_p7_split_merge(name, ps):
    _ok(P.pin_split_merge(oracle.decode, oracle.decode_partials,
                          oracle.merge_partials, oracle.reshape_and_cache,
                          SMALL[name], ps))


@pytest.mark.parametrize("name", list(SMALL))
def test_p8_contiguous(name):
    _ok(P.pin_contiguous(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


def test_p9_uncached_recompute():
    _ok(P.pin_uncached_recompute(oracle.decode, oracle.reshape_and_cache))


@pytest.mark.parametrize("name", list(SMALL))
def test_p10_sdpa(name):
    _ok(P.pin_sdpa(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


def test_p11_mpmath_tiny():
    _ok(P.pin_mpmath(oracle.decode, oracle.reshape_and_cache, W1))


@pytest.mark.parametrize("name", list(SMALL))
def test_p12_zero_scale(name):
    _ok(P.pin_zero_scale(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


@pytest.mark.parametrize("name", list(SMALL))
def test_p13_poison(name):
    _ok(P.pin_poison(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


@pytest.mark.parametrize("name", ["tiny_f32", "gqa4_bf16"])
def test_empty_sequence(name):
    _ok(P.pin_empty_sequence(oracle.decode, oracle.reshape_and_cache, SMALL[name]))


def test_merge_is_order_free():
    """Merging partitions in any order gives the same result (fp64 rounding)."""
    w = SMALL["gqa4_bf16"]
    inp = synth.make_inputs(w)
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    m, l, acc = oracle.decode_partials(inp["q"], k, v, inp["block_tables"],
                                       inp["context_lens"], inp["scale"], w.dtype, 16)
    perm = np.random.default_rng(5).permutation(m.shape[2])
    a = oracle.merge_partials(m, l, acc)
    b = oracle.merge_partials(m[:, :, perm], l[:, :, perm], acc[:, :, perm])
    assert np.max(np.abs(a - b)) <= 1e-13


# ------------------------------------------------------------ shared blocks
def _pairs(nb):
    # Sources and destinations disjoint; two pairs name blocks outside the pool.
    return np.array([[1, nb - 1], [3, 0], [-1, 2], [2, nb], [5, nb - 2]], dtype=np.int64)


@pytest.mark.parametrize("name", list(SMALL))
def test_p15_copy_blocks(name):
    inp = synth.make_inputs(SMALL[name])
    _ok(P.pin_copy_blocks(oracle.copy_blocks, inp, _pairs(inp["num_blocks"])))


@pytest.mark.parametrize("name,prefix_blocks", [("gqa4_bf16", 2), ("mha_f32", 1),
                                                ("mqa_bf16_bs32", 1)])
def test_p16_shared_prefix(name, prefix_blocks):
    w = SMALL[name]
    inp = synth.make_inputs(w)
    # Members: the sequences long enough to hold the shared prefix and a token.
    long_enough = inp["context_lens"] > prefix_blocks * w.block_size
    members = tuple(int(b) for b in np.nonzero(long_enough)[0])
    assert len(members) >= 2
    _ok(P.pin_shared_prefix(oracle.decode, oracle.reshape_and_cache, w, members,
                            prefix_blocks))


# ------------------------------------------------------------ prefill
PREFILL = {
    "pf_gqa2_bf16": synth.Workload("pf_gqa2_bf16", 3, 4, 2, 32, 16, "bf16",
                                   ("uniform", 20, 70), seed=31, query=("uniform", 1, 40)),
    "pf_full_f32": synth.Workload("pf_full_f32", 2, 2, 2, 16, 16, "f32",
                                  ("uniform", 10, 40), seed=32, query=("full",)),
    "pf_mqa_bf16_bs32": synth.Workload("pf_mqa_bf16_bs32", 2, 4, 1, 16, 32, "bf16",
                                       ("uniform", 30, 80), seed=33,
                                       query=("uniform", 1, 30)),
    "pf_full_gqa4_bf16": synth.Workload("pf_full_gqa4_bf16", 2, 8, 2, 32, 16, "bf16",
                                        ("uniform", 17, 50), seed=34, query=("full",)),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_p17_prefill_is_decode_per_token(name):
    inp = synth.make_prefill_inputs(PREFILL[name])
    _ok(P.pin_prefill_is_decode_per_token(oracle.prefill, oracle.decode,
                                          oracle.reshape_and_cache, inp))


@pytest.mark.parametrize("name", ["pf_full_f32", "pf_full_gqa4_bf16"])
def test_p18_prefill_causal_sdpa(name):
    inp = synth.make_prefill_inputs(PREFILL[name])
    _ok(P.pin_prefill_causal_sdpa(oracle.prefill, oracle.reshape_and_cache, inp))


@pytest.mark.parametrize("name", ["pf_full_f32", "pf_full_gqa4_bf16"])
def test_p19_prefill_chunk_equals_tail(name):
    inp = synth.make_prefill_inputs(PREFILL[name])
    tail = [5, 11]
    _ok(P.pin_prefill_chunk_equals_tail(oracle.prefill, oracle.reshape_and_cache, inp, tail))


@pytest.mark.parametrize("name", ["pf_gqa2_bf16", "pf_full_f32"])
def test_p20_prefill_first_token(name):
    _ok(P.pin_prefill_first_token(oracle.prefill, oracle.reshape_and_cache, PREFILL[name]))


def test_prefill_query_longer_than_context_is_nan():
    w = PREFILL["pf_gqa2_bf16"]
    inp = synth.make_prefill_inputs(w)
    start = inp["query_start"]
    ctx = inp["context_lens"].copy()
    ctx[1] = int(start[2] - start[1]) - 1
    out = oracle.prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                         ctx, start, inp["scale"], w.dtype)
    assert np.isnan(out[start[1]:start[2]]).all()
    assert np.isfinite(out[start[0]:start[1]]).all()
