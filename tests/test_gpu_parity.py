"""The HIP path against the float64 oracle on the GPU, through the C ABI.

Bit-exact: the KV write, the dense gather (block-table indexing), the
single-token and hard-max closed forms, block relabelling, NaN poisoning,
reruns.  Within tolerance (tests/_gpu.py: bf16 2e-3 + 1e-2|y| elementwise, max
abs 2e-3 below |y| = 0.5, max rel 1e-2 above |y| = 0.2; f32 1e-5 + 1e-5|y|):
every decode output against the oracle -- the two-launch step, the fused step
and graph replays of both.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import paged_kv_cache_reshape_amd as pa
from tests import _gpu as G
from tests import _pins as P

pytestmark = pytest.mark.gpu

ALL = ["tiny_f32", "qwen3_0p6b", "llama32_1b", "long_splitk", "mha_large", "mqa_large"]
# Small shapes that still span several blocks, partitions and a ragged tail.
EXTRA = {
    "f32_d128_bs32_g4": synth.Workload("f32_d128_bs32_g4", 5, 16, 4, 128, 32, "f32",
                                       ("uniform", 1, 700), num_blocks=160, seed=31),
    "bf16_d64_bs32_g8": synth.Workload("bf16_d64_bs32_g8", 7, 16, 2, 64, 32, "bf16",
                                       ("uniform", 1, 900), num_blocks=260, seed=32),
    "bf16_d128_bs16_g16": synth.Workload("bf16_d128_bs16_g16", 6, 32, 2, 128, 16,
                                         "bf16", ("uniform", 1, 1500), seed=33),
    "f32_d64_bs16_g1": synth.Workload("f32_d64_bs16_g1", 9, 4, 4, 64, 16, "f32",
                                      ("uniform", 1, 300), seed=34),
    "bf16_d64_bs16_g2": synth.Workload("bf16_d64_bs16_g2", 11, 8, 4, 64, 16, "bf16",
                                       ("uniform", 1, 2000), seed=35),
    "bf16_d128_bs32_g2": synth.Workload("bf16_d128_bs32_g2", 5, 8, 4, 128, 32, "bf16",
                                        ("uniform", 1, 700), num_blocks=120, seed=36),
    "bf16_d64_bs32_g4": synth.Workload("bf16_d64_bs32_g4", 6, 16, 4, 64, 32, "bf16",
                                       ("uniform", 1, 900), num_blocks=200, seed=37),
    "bf16_d128_bs16_g4": synth.Workload("bf16_d128_bs16_g4", 6, 16, 4, 128, 16, "bf16",
                                        ("uniform", 1, 1500), seed=38),
    # 32 query heads per kv head over 32-token blocks: the 32x32-tile decode.
    "bf16_d64_bs32_g32": synth.Workload("bf16_d64_bs32_g32", 7, 64, 2, 64, 32, "bf16",
                                        ("uniform", 1, 1200), seed=39),
}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def inputs_for(name, **kw):
    if name in EXTRA:
        return synth.make_inputs(EXTRA[name], **kw)
    if not kw:
        return G.cached_inputs(name)
    return synth.make_inputs(synth.WORKLOADS[name], **kw)


def gpu_step(d, partition_size=0, write=True):
    """One step on the GPU: the KV write, then decode.  Returns out (device)."""
    if write:
        pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"],
                             d["slot_mapping"])
    return pa.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"],
                                     d["block_tables"], d["context_lens"], d["scale"],
                                     partition_size=partition_size)


def oracle_step(inp, seqs=None):
    """The oracle's write + decode, optionally on a subset of sequences."""
    w = inp["workload"]
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    sel = slice(None) if seqs is None else np.asarray(seqs)
    out = oracle.decode(inp["q"][sel], k, v, inp["block_tables"][sel],
                        inp["context_lens"][sel], inp["scale"], w.dtype)
    return out, (k, v)


# ------------------------------------------------------------------ KV write
@pytest.mark.parametrize("name", ALL)
def test_write_bit_exact(name):
    inp = inputs_for(name)
    w = inp["workload"]
    say("reshape_and_cache", name, w)
    d = G.upload(inp)
    slots = inp["slot_mapping"].copy()
    slots[0] = -1                                 # padding row: skipped
    if len(slots) > 2:
        slots[1] = inp["num_blocks"] * w.block_size  # past the pool: skipped
    d["slot_mapping"] = torch.from_numpy(slots).cuda()
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"],
                         d["slot_mapping"])
    torch.cuda.synchronize()
    oslots = slots.copy()
    oslots[oslots >= inp["num_blocks"] * w.block_size] = -1
    k_ref, v_ref = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                            inp["v_cache"], oslots)
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    assert np.array_equal(G.host_storage(d["v_cache"]), v_ref)


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("f32", 2, 64),
                                         ("bf16", 1, 64)])
def test_write_many_tokens(dtype, hkv, d):
    """A prefill-sized write (N >> B): 3000 distinct slots in a 400-block pool."""
    rng = np.random.default_rng(77)
    nb, bs, n = 400, 16, 3000
    say("reshape_and_cache many", dtype, hkv, d)
    shape = (nb, bs, hkv, d)
    kc = synth._draw(rng, shape, 1.0, dtype)
    vc = synth._draw(rng, shape, 1.0, dtype)
    key = synth._draw(rng, (n, hkv, d), 1.0, dtype)
    val = synth._draw(rng, (n, hkv, d), 1.0, dtype)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[::97] = -1
    dk, dv = G.dev_tensor(kc, dtype), G.dev_tensor(vc, dtype)
    pa.reshape_and_cache(G.dev_tensor(key, dtype), G.dev_tensor(val, dtype), dk, dv,
                         torch.from_numpy(slots).cuda())
    k_ref, v_ref = oracle.reshape_and_cache(key, val, kc, vc, slots)
    assert np.array_equal(G.host_storage(dk), k_ref)
    assert np.array_equal(G.host_storage(dv), v_ref)


# ------------------------------------------------------------------ gather
@pytest.mark.parametrize("name", ALL + list(EXTRA))
def test_gather_bit_exact(name):
    inp = inputs_for(name)
    say("debug_gather_kv", name)
    d = G.upload(inp)
    nseq = 24 if name in ("mha_large", "mqa_large") else None
    bt, cl = d["block_tables"], d["context_lens"]
    if nseq:
        bt, cl = bt[:nseq].contiguous(), cl[:nseq].contiguous()
    kd, vd = pa.debug_gather_kv(d["k_cache"], d["v_cache"], bt, cl)
    tables = inp["block_tables"][:nseq] if nseq else inp["block_tables"]
    lens = inp["context_lens"][:nseq] if nseq else inp["context_lens"]
    assert np.array_equal(G.host_storage(kd), oracle.gather_kv(inp["k_cache"], tables, lens))
    assert np.array_equal(G.host_storage(vd), oracle.gather_kv(inp["v_cache"], tables, lens))


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_0p6b", "llama32_1b", "mha_large",
                                  "mqa_large"] + list(EXTRA))
def test_decode_matches_oracle(name):
    inp = inputs_for(name)
    w = inp["workload"]
    say("write+decode", name, "partition", w.partition_size)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, w.partition_size))
    ref, (k_ref, v_ref) = oracle_step(inp)
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    G.assert_close(out, ref, w.dtype, name)


@pytest.mark.parametrize("name", ["qwen3_0p6b", "llama32_1b", "bf16_d64_bs32_g4",
                                  "bf16_d128_bs16_g4", "f32_d64_bs16_g1", "bf16_d64_bs16_g2"])
def test_fixed_schedule_matches_oracle(name, monkeypatch):
    """The fixed schedule (library partition sizes) on shapes the balanced
    schedule takes by default: the vector-ALU kernel at 1 or 2 query heads
    per kv head, the matrix-core kernel at 4."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "fixed")
    inp = inputs_for(name)
    w = inp["workload"]
    say("write+decode (fixed schedule)", name)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, 0))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, w.dtype, name)


@pytest.mark.parametrize("name", ["mqa_large", "bf16_d64_bs32_g8", "bf16_d128_bs16_g16",
                                  "llama32_1b", "bf16_d64_bs32_g4", "bf16_d128_bs16_g4"])
def test_vector_alu_kernel_matches_oracle(name, monkeypatch):
    """The vector-ALU kernel on shapes the matrix-core kernel takes by default."""
    G.setopt(monkeypatch, "PAGEDATTN_DECODE_KERNEL", "valu")
    inp = inputs_for(name)
    w = inp["workload"]
    say("write+decode (vector ALU kernel)", name)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, w.partition_size))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, w.dtype, name)


@pytest.mark.parametrize("name", ["qwen3_0p6b", "bf16_d128_bs16_g16", "bf16_d64_bs32_g8"])
@pytest.mark.parametrize("factor", [4.0, 16.0])
def test_large_scores_match_oracle(name, factor):
    """Scores several times wider than 1/sqrt(D) gives: the running maximum
    moves often, in every tile, and the kept maximum is rescaled many times."""
    inp = dict(inputs_for(name))
    w = inp["workload"]
    inp["scale"] = np.float32(inp["scale"] * factor)
    say("decode scale x", factor, name)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, w.partition_size))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, w.dtype, f"{name} scale x{factor}")


@pytest.fixture(scope="module")
def long_splitk_oracle():
    """The oracle's write + decode of every sequence of the 32,768-token batch
    (it gathers one sequence at a time, so each sequence's float64 rows are
    freed before the next is read)."""
    inp = inputs_for("long_splitk")
    ref, _ = oracle_step(inp)
    return inp, ref


@pytest.mark.parametrize("ps", [512, 0])
def test_decode_long_split_k(long_splitk_oracle, ps):
    """32,768-token sequences at 512-token partitions as stated (64 per
    sequence) and at the library's choice: split sequences of 16 or more
    partitions are merged by the merge kernel that follows the partition
    launch.  Every output row of all eight sequences against the oracle."""
    inp, ref = long_splitk_oracle
    w = inp["workload"]
    say("write+decode long_splitk partition", ps or "library choice")
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, ps))
    G.assert_close(out, ref, w.dtype, f"long_splitk ps={ps}")
    # The fused step, the launch the benchmark times, on fresh caches.
    d2 = G.upload(inp)
    got = G.host_f64(fused_step(d2, ps))
    G.assert_close(got, ref, w.dtype, f"long_splitk fused step ps={ps}")


@pytest.mark.parametrize("merge", ["inkernel", "separate"])
@pytest.mark.parametrize("name,ps", [("f32_d128_bs32_g4", 64), ("bf16_d128_bs16_g16", 128),
                                     ("bf16_d64_bs16_g2", 256), ("bf16_d64_bs32_g8", 64),
                                     ("llama32_1b", 512), ("bf16_d64_bs32_g32", 64)])
def test_merge_paths_match_oracle(name, ps, merge, monkeypatch):
    """Split sequences merged by the last partition workgroup to arrive, or by
    the merge kernel that follows the partition launch."""
    G.setopt(monkeypatch, "PAGEDATTN_MERGE", merge)
    inp = inputs_for(name)
    w = inp["workload"]
    say("write+decode", name, "partition", ps, "merge", merge)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, ps))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, w.dtype, f"{name} ps={ps} merge={merge}")


@pytest.mark.parametrize("merge", ["inkernel", "separate"])
@pytest.mark.parametrize("hpw", [1, 2, 4])
@pytest.mark.parametrize("name,ps", [("f32_d128_bs32_g4", 64), ("bf16_d128_bs32_g2", 64),
                                     ("bf16_d64_bs16_g2", 256)])
def test_heads_per_workgroup_match_oracle(name, ps, hpw, merge, monkeypatch):
    """Workgroups forced to take 1, 2 or 4 kv heads; split sequences merged by
    the last partition to arrive (every kv head of its group in one pass, a
    separate code path for each group size) or by the merge kernel."""
    monkeypatch.setenv("PAGEDATTN_HEADS_PER_WG", str(hpw))
    G.setopt(monkeypatch, "PAGEDATTN_MERGE", merge)
    inp = inputs_for(name)
    w = inp["workload"]
    say("write+decode", name, "partition", ps, "heads per workgroup", hpw, "merge", merge)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, ps))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, w.dtype, f"{name} ps={ps} hpw={hpw} merge={merge}")


@pytest.mark.parametrize("G_", [4, 8, 16, 32])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_matrix_core_kernel_every_shape(D, bs, G_):
    """Every (head_dim, block size, group) the matrix-core kernel is built
    for, on a small ragged batch that splits its longer sequences."""
    hkv = 2 if G_ <= 16 else 1
    w = synth.Workload(f"mfma_d{D}_bs{bs}_g{G_}", 4, G_ * hkv, hkv, D, bs, "bf16",
                       ("uniform", 1, 600), seed=40 + D + bs + G_)
    inp = synth.make_inputs(w)
    say("write+decode", w.name, "partition 128")
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, 128))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, "bf16", w.name)


@pytest.mark.parametrize("G_", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vector_kernel_every_shape(dtype, D, bs, G_, monkeypatch):
    """Every (dtype, head_dim, block size, group) the vector-ALU kernel is
    built for (forced where the matrix cores would take the shape), on a
    small ragged batch that splits its longer sequences."""
    G.setopt(monkeypatch, "PAGEDATTN_DECODE_KERNEL", "valu")
    hkv = 2 if G_ <= 16 else 1
    w = synth.Workload(f"valu_{dtype}_d{D}_bs{bs}_g{G_}", 4, G_ * hkv, hkv, D, bs, dtype,
                       ("uniform", 1, 600), seed=60 + D + bs + G_)
    inp = synth.make_inputs(w)
    say("write+decode (vector ALU kernel)", w.name, "partition 128")
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, 128))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, dtype, w.name)


@pytest.mark.parametrize("ps", [16, 64, 256, 1024, 1040, 2048])
def test_partition_sizes_agree(ps):
    inp = inputs_for("qwen3_0p6b")
    say("decode qwen3 partition", ps)
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, ps))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, "bf16", f"partition {ps}")


def test_max_context_everywhere():
    """Every sequence fills its whole table (2048 tokens = 128 blocks); every
    row of all 32 sequences against the oracle."""
    w = synth.WORKLOADS["qwen3_0p6b"]
    inp = synth.make_inputs(w, context_lens=np.full(w.num_seqs, 2048, np.int32))
    say("decode qwen3 ctx=2048 all")
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d))
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, "bf16", "max ctx")
    d2 = G.upload(inp)
    G.assert_close(G.host_f64(fused_step(d2)), ref, "bf16", "max ctx fused step")


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_0p6b", "bf16_d64_bs32_g8",
                                  "f32_d128_bs32_g4", "mqa_large", "bf16_d128_bs32_g2",
                                  "bf16_d64_bs32_g4"])
def test_single_token_exact(name):
    """P3 on the GPU: one cached token -> out is exactly that V row."""
    w = EXTRA.get(name) or synth.WORKLOADS[name]
    inp = synth.make_inputs(w, context_lens=np.ones(w.num_seqs, dtype=np.int32))
    say("decode ctx=1", name)
    d = G.upload(inp)
    out = G.host_storage(gpu_step(d))
    _, (k_ref, v_ref) = oracle_step(inp)
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        vrow = v_ref[int(inp["block_tables"][b, 0]), 0]
        expect = np.repeat(vrow, grp, axis=0)  # head h reads kv head h // grp
        assert np.array_equal(out[b], expect), b


ONEHOT = {
    "gqa4_bf16": synth.Workload("gqa4_bf16", 6, 8, 2, 64, 16, "bf16", ("uniform", 1, 100),
                                num_blocks=48, seed=21),
    "gqa8_bf16": synth.Workload("gqa8_bf16", 4, 16, 2, 128, 32, "bf16", ("uniform", 1, 100),
                                num_blocks=24, seed=22),
    "mqa16_bf16": synth.Workload("mqa16_bf16", 5, 16, 1, 64, 16, "bf16", ("uniform", 1, 120),
                                 num_blocks=48, seed=23),
}


@pytest.mark.parametrize("name", ["tiny_f32"] + list(ONEHOT))
def test_onehot_exact(name):
    """P4 on the GPU: scale 1e5 -> out is exactly V of the top-scoring row."""
    w = synth.WORKLOADS["tiny_f32"] if name == "tiny_f32" else ONEHOT[name]
    inp, (k, v), best = P.onehot_inputs(w)
    say("decode one-hot", name)
    d = G.upload(inp)
    d["k_cache"] = G.dev_tensor(k, w.dtype)
    d["v_cache"] = G.dev_tensor(v, w.dtype)
    d["scale"] = 1e5
    out = G.host_f64(gpu_step(d, write=False))
    for (b, h), row in best.items():
        assert np.array_equal(out[b, h], row), (b, h)


def test_block_relabelling_bit_identical():
    """P5 on the GPU: permuting physical ids (table updated) changes no bit."""
    inp = inputs_for("qwen3_0p6b")
    say("decode qwen3 relabelled")
    d = G.upload(inp)
    base = G.host_storage(gpu_step(d))
    rng = np.random.default_rng(5)
    perm = rng.permutation(inp["num_blocks"])
    k, v = G.host_storage(d["k_cache"]), G.host_storage(d["v_cache"])
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm], v2[perm] = k, v
    t = inp["block_tables"]
    t2 = np.where(t >= 0, perm[np.clip(t, 0, None)], t).astype(np.int32)
    d2 = dict(d, k_cache=G.dev_tensor(k2, "bf16"), v_cache=G.dev_tensor(v2, "bf16"),
              block_tables=torch.from_numpy(t2).cuda())
    assert np.array_equal(G.host_storage(gpu_step(d2, write=False)), base)


def test_mqa_equals_replicated_mha():
    """P6 on the GPU: the MQA batch equals MHA over the KV head copied 32x."""
    inp = inputs_for("mqa_large")
    say("decode mqa vs replicated mha")
    d = G.upload(inp)
    mqa = G.host_f64(gpu_step(d))
    k = d["k_cache"].repeat_interleave(32, dim=2).contiguous()
    v = d["v_cache"].repeat_interleave(32, dim=2).contiguous()
    mha = G.host_f64(pa.paged_attention_decode(d["q"], k, v, d["block_tables"],
                                               d["context_lens"], d["scale"]))
    ref, _ = oracle_step(inp)
    G.assert_close(mqa, ref, "bf16", "mqa")
    G.assert_close(mha, ref, "bf16", "replicated mha")


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_0p6b", "bf16_d64_bs32_g8",
                                  "bf16_d128_bs32_g2", "bf16_d64_bs32_g4"])
def test_nan_poison_bit_identical(name):
    """P13 on the GPU: NaN in unread slots and poison-padded tables change no bit."""
    w = EXTRA.get(name) or synth.WORKLOADS[name]
    clean = synth.make_inputs(w)
    dirty = synth.make_inputs(w, poison=True)
    say("decode poison", name)
    a = G.host_storage(gpu_step(G.upload(clean)))
    b = G.host_storage(gpu_step(G.upload(dirty)))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,ps", [("qwen3_0p6b", 64), ("qwen3_0p6b", 256), ("long_splitk", 512),
                                     ("bf16_d128_bs16_g16", 128), ("bf16_d128_bs16_g16", 32)])
def test_rerun_bit_identical(name, ps):
    """P14: partitions finish in any order, the merge does not depend on it."""
    inp = inputs_for(name)
    say("decode rerun", name, ps)
    d = G.upload(inp)
    a = G.host_storage(gpu_step(d, ps))
    for _ in range(3):
        b = G.host_storage(gpu_step(d, ps, write=False))
        assert np.array_equal(a, b)


def test_empty_sequences_give_zero_rows():
    w = synth.WORKLOADS["qwen3_0p6b"]
    ctx = G.cached_inputs("qwen3_0p6b")["context_lens"].copy()
    ctx[[0, 5, 31]] = 0
    inp = synth.make_inputs(w, context_lens=ctx)
    say("decode with empty sequences")
    d = G.upload(inp)
    out = G.host_f64(gpu_step(d, 64))
    assert np.all(out[[0, 5, 31]] == 0)
    ref, _ = oracle_step(inp)
    G.assert_close(out, ref, "bf16", "empty rows")


@pytest.mark.parametrize("merge", ["inkernel", "separate"])
@pytest.mark.parametrize("name,ps", [("qwen3_0p6b", 256), ("bf16_d128_bs16_g16", 128)])
def test_bad_table_entries_give_nan_rows_only(name, ps, merge, monkeypatch):
    """A block id outside the pool, or a length past the table, is never
    dereferenced: that sequence's rows become NaN, the others are unchanged
    (with split sequences merged in the partition kernel or after it; the
    vector-ALU kernel and the matrix-core one)."""
    G.setopt(monkeypatch, "PAGEDATTN_MERGE", merge)
    inp = inputs_for(name)
    w = inp["workload"]
    B, bs = w.num_seqs, w.block_size
    say("decode bad table entries", name, "partition", ps, "merge", merge)
    d = G.upload(inp)
    base = G.host_storage(gpu_step(d, ps))
    t = inp["block_tables"].copy()
    ctx = inp["context_lens"].copy()
    bad = [1, B // 2, B - 1]
    t[bad[0], 0] = inp["num_blocks"]                  # one past the pool
    t[bad[1], (ctx[bad[1]] - 1) // bs] = -5           # negative, in the last used block
    ctx[bad[2]] = (t.shape[1] + 1) * bs               # longer than the table
    d2 = dict(d, block_tables=torch.from_numpy(t).cuda(),
              context_lens=torch.from_numpy(ctx).cuda())
    out = gpu_step(d2, ps, write=False)
    got = G.host_f64(out)
    assert np.all(np.isnan(got[bad]))
    keep = [b for b in range(B) if b not in bad]
    assert np.array_equal(G.host_storage(out)[keep], base[keep])


# ------------------------------------------------------------------ fused step
def fused_step(d, partition_size=0):
    return pa.decode_step(d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"],
                          d["block_tables"], d["context_lens"], d["scale"],
                          partition_size=partition_size)


@pytest.mark.parametrize("name,ps", [("qwen3_0p6b", 0), ("qwen3_0p6b", 64), ("tiny_f32", 0),
                                     ("llama32_1b", 0), ("mqa_large", 0), ("mqa_large", 256),
                                     ("bf16_d64_bs32_g32", 96),
                                     ("bf16_d128_bs16_g16", 128), ("bf16_d128_bs16_g16", 32),
                                     ("bf16_d64_bs32_g8", 0), ("f32_d128_bs32_g4", 64)])
def test_decode_step_equals_write_then_decode(name, ps):
    """The fused step (write of each sequence's token at position L - 1 inside
    the decode launch) gives the bits of the two calls: the output and both
    caches, in both kernels and with either merge path."""
    inp = inputs_for(name)
    say("fused step", name, ps)
    d1, d2 = G.upload(inp), G.upload(inp)
    want = G.host_storage(gpu_step(d1, ps))
    got_dev = fused_step(d2, ps)
    got = G.host_storage(got_dev)
    assert np.array_equal(got, want)
    for c in ("k_cache", "v_cache"):
        assert torch.equal(d1[c], d2[c]), c
    # And against the oracle directly: its write, then its decode.
    ref, (k_ref, v_ref) = oracle_step(inp)
    G.assert_close(G.host_f64(got_dev), ref, inp["workload"].dtype, f"fused step {name}")
    assert np.array_equal(G.host_storage(d2["k_cache"]), k_ref)
    assert np.array_equal(G.host_storage(d2["v_cache"]), v_ref)


@pytest.mark.parametrize("name,ps", [("qwen3_0p6b", 0), ("qwen3_0p6b", 64), ("tiny_f32", 0),
                                     ("llama32_1b", 0), ("bf16_d64_bs32_g8", 0),
                                     ("bf16_d64_bs32_g32", 96), ("f32_d128_bs32_g4", 64),
                                     ("mha_large", 0), ("mqa_large", 0)])
def test_decode_step_target_slot_holds_nan(name, ps):
    """The slot a step writes holds anything beforehand (a fresh block is
    uninitialised memory): NaN there changes no bit of the fused step's output,
    also where the new token is the first of its block, whose rows past the
    context load that slot and are masked; afterwards both caches equal the
    separate write's.  Every schedule and kernel family, full-size batches
    included (the fixed kernels copy the rows in extra workgroups that may
    run while the token's partition reads the slot)."""
    base = inputs_for(name)
    w = base["workload"]
    bs = w.block_size
    ctx = base["context_lens"].copy()
    ctx[0], ctx[1] = bs + 1, 1                   # new token first in its block
    if len(ctx) > 2:
        ctx[2] = min(2 * bs + 1, w.max_blocks_per_seq * bs)
    inp = inputs_for(name, context_lens=ctx)
    say("fused step, NaN in the target slot", name, ps)
    d1, d2 = G.upload(inp), G.upload(inp)
    want = G.host_storage(gpu_step(d1, ps))
    nan = torch.tensor(float("nan"), dtype=d2["k_cache"].dtype, device="cuda")
    slots = torch.from_numpy(inp["slot_mapping"]).cuda()
    slots = slots[slots >= 0]
    for c in ("k_cache", "v_cache"):
        flat = d2[c].view(-1, *d2[c].shape[2:])
        flat[slots] = nan
    got = G.host_storage(fused_step(d2, ps))
    assert np.array_equal(got, want)
    for c in ("k_cache", "v_cache"):
        assert torch.equal(d1[c], d2[c]), c


def test_decode_step_edge_sequences():
    """Empty sequences, a new token whose block lies outside the pool and a
    length past the table write nothing; their rows are what the decode
    gives (zeros, NaN), every other row and slot is the two calls' result;
    a sequence of one token sees only the token just written."""
    w = synth.WORKLOADS["qwen3_0p6b"]
    ctx = G.cached_inputs("qwen3_0p6b")["context_lens"].copy()
    ctx[[0, 5]] = 0
    ctx[9] = 1
    inp = synth.make_inputs(w, context_lens=ctx)
    t = inp["block_tables"].copy()
    c = inp["context_lens"].copy()
    t[7, (c[7] - 1) // 16] = inp["num_blocks"] + 3   # the new token's block: outside the pool
    c[11] = (t.shape[1] + 1) * 16                    # past the table
    slots = inp["slot_mapping"].copy()
    slots[[7, 11]] = -1                              # what the fused step writes for them
    say("fused step edge sequences")
    d1, d2 = G.upload(inp), G.upload(inp)
    for d in (d1, d2):
        d["block_tables"] = torch.from_numpy(t).cuda()
        d["context_lens"] = torch.from_numpy(c).cuda()
    d1["slot_mapping"] = torch.from_numpy(slots).cuda()
    want = G.host_storage(gpu_step(d1, 256))
    got_dev = fused_step(d2, 256)
    assert np.array_equal(G.host_storage(got_dev), want)
    for name in ("k_cache", "v_cache"):
        assert torch.equal(d1[name], d2[name]), name
    got = G.host_f64(got_dev)
    assert np.all(got[[0, 5]] == 0) and np.all(np.isnan(got[[7, 11]]))
    ref, _ = oracle_step(inp, seqs=[9])
    G.assert_close(got[[9]], ref, "bf16", "one-token sequence")


def test_side_stream_and_given_out():
    """Work goes on the caller's current stream; `out` may be supplied."""
    inp = inputs_for("qwen3_0p6b")
    say("decode on side stream")
    d = G.upload(inp)
    base = G.host_storage(gpu_step(d))
    s = torch.cuda.Stream()
    out = torch.full_like(d["q"], float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pa.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["context_lens"], d["scale"], out=out)
    s.synchronize()
    assert np.array_equal(G.host_storage(out), base)


def test_one_workspace_serves_both_schedules():
    """One workspace and one counter array shared by calls that lay partial
    states out differently: the balanced schedule (vector-ALU and matrix-core
    workers, whose merges take a zero word for "not stored yet") alternating
    with fixed partitions (merged in the launch, or by the merge kernel at 16
    or more partitions).  Every call must leave the workspace all zero, or a
    later balanced call would read a stale state as stored."""
    cases = [("qwen3_0p6b", 0), ("qwen3_0p6b", 64), ("llama32_1b", 0), ("qwen3_0p6b", 256),
             ("bf16_d128_bs16_g16", 32), ("qwen3_0p6b", 0), ("llama32_1b", 0),
             ("llama32_1b", 128)]
    need = 256
    for name, ps in cases:
        w = inputs_for(name)["workload"]
        need = max(need, pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                   w.head_dim, inputs_for(name)["max_blocks"],
                                                   w.block_size, ps))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for name, ps in cases:
        inp = inputs_for(name)
        w = inp["workload"]
        say("shared workspace", name, "partition", ps or "library choice")
        d = G.upload(inp)
        out = pa.decode_step(d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"],
                             d["block_tables"], d["context_lens"], d["scale"],
                             partition_size=ps, workspace=ws, counters=cnt)
        ref, _ = oracle_step(inp)
        G.assert_close(G.host_f64(out), ref, w.dtype, f"{name} ps={ps}")
        assert int(cnt.abs().sum()) == 0
        assert int(ws.count_nonzero()) == 0, f"{name} ps={ps}: the workspace is left all zero"


def test_one_counter_array_serves_every_geometry(monkeypatch):
    """Counters left at zero by each call: alternate two geometries whose
    partial results overlap differently, with one shared counter array
    (merged in the partition kernel, the path that counts arrivals)."""
    G.setopt(monkeypatch, "PAGEDATTN_MERGE", "inkernel")
    cnt = torch.zeros(4096, dtype=torch.int32, device="cuda")
    cases = [("qwen3_0p6b", 64), ("bf16_d128_bs16_g16", 32), ("llama32_1b", 128),
             ("qwen3_0p6b", 32)]
    for name, ps in cases:
        inp = inputs_for(name)
        w = inp["workload"]
        say("decode shared counters", name, ps)
        d = G.upload(inp)
        pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"],
                             d["slot_mapping"])
        need = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                         w.head_dim, inp["max_blocks"], w.block_size, ps)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        out = pa.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"],
                                        d["block_tables"], d["context_lens"], d["scale"],
                                        partition_size=ps, workspace=ws, counters=cnt)
        ref, _ = oracle_step(inp)
        G.assert_close(G.host_f64(out), ref, w.dtype, f"{name} ps={ps}")
        assert int(cnt.abs().sum()) == 0
        assert int(ws.count_nonzero()) == 0, "the workspace is left all zero"


# ------------------------------------------------------------------ stream schedule
def stream_case(dtype, D, bs, G_, hkv=2, B=9, top=900, seed=0, empty=True):
    w = synth.Workload(f"stream_{dtype}_d{D}_bs{bs}_g{G_}_{seed}", B, G_ * hkv, hkv, D, bs,
                       dtype, ("uniform", 1, top), seed=500 + seed + D + bs + G_)
    inp = synth.make_inputs(w)
    if empty:
        ctx = inp["context_lens"].copy()
        ctx[::4] = [0, 1, 17][: len(ctx[::4])] + [1] * max(0, len(ctx[::4]) - 3)
        inp = synth.make_inputs(w, context_lens=ctx)
    return inp


def check_stream(inp, what):
    """Write + decode and the fused step against the oracle; the two agree
    bit for bit (output and caches)."""
    w = inp["workload"]
    d1, d2 = G.upload(inp), G.upload(inp)
    out = gpu_step(d1)
    ref, (k_ref, v_ref) = oracle_step(inp)
    G.assert_close(G.host_f64(out), ref, w.dtype, what)
    got = fused_step(d2)
    assert np.array_equal(G.host_storage(got), G.host_storage(out)), what
    assert torch.equal(d1["k_cache"], d2["k_cache"]) and torch.equal(d1["v_cache"], d2["v_cache"])
    assert np.array_equal(G.host_storage(d2["k_cache"]), k_ref)
    return out


@pytest.mark.parametrize("workers", [8, 64, 1024])
@pytest.mark.parametrize("G_", [1, 2, 4])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stream_schedule_every_shape(dtype, D, bs, G_, workers, monkeypatch):
    """The balanced schedule on every (dtype, head_dim, block size, group) it
    is built for, on a ragged batch with empty and one-token sequences: with
    few workers (ranges of up to 128 blocks, many sequences each), some, and
    many (sequences split over many workers, merged by the last to finish)."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", workers)
    inp = stream_case(dtype, D, bs, G_)
    say("stream", inp["workload"].name, "workers", workers)
    check_stream(inp, f"stream {inp['workload'].name} workers={workers}")


@pytest.mark.parametrize("merge", ["separate", "inkernel"])
@pytest.mark.parametrize("shape", [("bf16", 128, 16, 2, 64), ("f32", 64, 32, 1, 8),
                                   ("bf16", 64, 32, 4, 1024), ("bf16", 128, 16, 2, 4096)])
def test_stream_merge_paths(shape, merge, monkeypatch):
    """Split sequences of the balanced schedule merged by the last worker to
    finish, or by the merge kernel launched after the stream kernel."""
    dtype, D, bs, G_, workers = shape
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", workers)
    G.setopt(monkeypatch, "PAGEDATTN_MERGE", merge)
    inp = stream_case(dtype, D, bs, G_, seed=3)
    say("stream merge", merge, inp["workload"].name, "workers", workers)
    check_stream(inp, f"stream merge={merge} {inp['workload'].name}")


def test_stream_one_long_sequence_many_pieces(monkeypatch):
    """A 4096-token sequence among short ones, 2048 workers per kv head: it
    splits into dozens of pieces (merged four at a time)."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", 4096)
    w = synth.Workload("stream_long_one", 6, 16, 8, 128, 16, "bf16", ("uniform", 1, 4096),
                       seed=71)
    ctx = np.array([4096, 3, 200, 1, 0, 77], dtype=np.int32)
    inp = synth.make_inputs(w, context_lens=ctx)
    say("stream one long sequence")
    check_stream(inp, "stream long one")


def test_stream_many_short_sequences(monkeypatch):
    """2000 sequences of 0-16 tokens, 16 workers per kv head: a worker's range
    spans more than 64 sequences (the range set-up walks the sequence starts
    in chunks of 64)."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", 32)
    w = synth.Workload("stream_many_short", 2000, 4, 2, 64, 16, "bf16", ("uniform", 0, 16),
                       seed=72)
    inp = synth.make_inputs(w)
    say("stream 2000 short sequences")
    check_stream(inp, "stream many short")


@pytest.mark.parametrize("hq,hkv,d", [(8, 4, 128), (16, 4, 64)])
@pytest.mark.parametrize("B", [63, 64, 65])
def test_stream_set_up_either_side_of_64_sequences(B, hq, hkv, d, monkeypatch):
    """Up to 64 sequences the balanced schedule sets ranges up in each wave's
    registers, above that through LDS: both workers (G = 2 vector ALU, G = 4
    matrix cores) against the oracle, with empty
    sequences first, last and in between (ranges of a few blocks, so every
    range's start falls in a different place)."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", 512)
    rng = np.random.default_rng(1064 + B)
    ctx = rng.integers(1, 700, size=B).astype(np.int32)
    ctx[[0, B // 3, B - 1]] = 0
    w = synth.Workload(f"stream_b{B}_g{hq // hkv}", B, hq, hkv, d, 16, "bf16",
                       ("uniform", 1, 700), seed=64 + B)
    inp = synth.make_inputs(w, context_lens=ctx)
    say("stream set-up", B, "sequences, G", hq // hkv, "D", d)
    check_stream(inp, f"stream B={B} G={hq // hkv} D={d}")


@pytest.mark.parametrize("name", ["qwen3_0p6b", "llama32_1b"])
def test_stream_library_choice(name):
    """The library's own choice for the Qwen3- and Llama-3.2-shaped batches is
    the balanced schedule (reported as partition size 0; the vector-ALU and
    the matrix-core worker), and its result is the oracle's."""
    w = synth.WORKLOADS[name]
    assert pa.decode_partition_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.max_blocks_per_seq, w.block_size, 0) == 0
    say("stream library choice", name)
    check_stream(inputs_for(name), f"stream {name}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32])
def test_stream_vector_worker_at_four_heads(D, bs, monkeypatch):
    """The vector-ALU worker on bfloat16 with 4 query heads per kv head (the
    matrix-core worker's shapes), forced."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    G.setopt(monkeypatch, "PAGEDATTN_DECODE_KERNEL", "valu")
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", 64)
    inp = stream_case("bf16", D, bs, 4, seed=5)
    say("stream vector worker G=4", inp["workload"].name)
    check_stream(inp, f"stream valu {inp['workload'].name}")


@pytest.mark.parametrize("name", ["qwen3_0p6b", "llama32_1b"])
def test_stream_bad_table_entries(name, monkeypatch):
    """Block ids outside the pool on the balanced schedule (both workers):
    those sequences' rows are NaN, nothing is dereferenced, every other row
    keeps its bits (the lengths, hence the ranges, are unchanged); a length
    past the table gives NaN rows too."""
    G.setopt(monkeypatch, "PAGEDATTN_SCHEDULE", "stream")
    inp = inputs_for(name)
    w = inp["workload"]
    B, bs = w.num_seqs, w.block_size
    say("stream bad table entries", name)
    d = G.upload(inp)
    base = G.host_storage(gpu_step(d))
    t = inp["block_tables"].copy()
    ctx = inp["context_lens"].copy()
    bad = [2, B // 2 + 1, B - 2]
    t[bad[0], 0] = inp["num_blocks"]
    t[bad[1], (ctx[bad[1]] - 1) // bs] = -5
    t[bad[2], (ctx[bad[2]] - 1) // (2 * bs)] = inp["num_blocks"] + 100
    d2 = dict(d, block_tables=torch.from_numpy(t).cuda())
    out = gpu_step(d2, write=False)
    assert np.all(np.isnan(G.host_f64(out)[bad]))
    keep = [b for b in range(B) if b not in bad]
    assert np.array_equal(G.host_storage(out)[keep], base[keep])
    ctx2 = ctx.copy()
    ctx2[5] = (t.shape[1] + 1) * bs
    d3 = dict(d, context_lens=torch.from_numpy(ctx2).cuda())
    got = G.host_f64(gpu_step(d3, write=False))
    assert np.all(np.isnan(got[5]))
    inp2 = dict(inp, context_lens=ctx2)
    k, v = G.host_storage(d["k_cache"]), G.host_storage(d["v_cache"])
    keep = [b for b in range(B) if b != 5]
    ref = oracle.decode(inp["q"][keep], k, v, inp["block_tables"][keep], ctx2[keep],
                        inp["scale"], "bf16")
    G.assert_close(got[keep], ref, "bf16", "stream, one length past the table")


def test_stream_rerun_bit_identical_and_counters_zero(monkeypatch):
    """Reruns give the same bits whatever order the workers finish in, and
    every call leaves the arrival counters at zero."""
    G.setopt(monkeypatch, "PAGEDATTN_STREAM_WORKERS", 2048)
    inp = inputs_for("qwen3_0p6b")
    w = inp["workload"]
    say("stream rerun")
    d = G.upload(inp)
    cnt = torch.zeros(w.num_seqs * w.num_kv_heads, dtype=torch.int32, device="cuda")
    need = pa.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                     inp["max_blocks"], w.block_size, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(4):
        outs.append(G.host_storage(pa.decode_step(
            d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"], d["block_tables"],
            d["context_lens"], d["scale"], workspace=ws, counters=cnt)))
        torch.cuda.synchronize()
        assert int(cnt.abs().sum()) == 0
        assert int(ws.count_nonzero()) == 0, "the workspace is left all zero"
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ------------------------------------------------------------------ shared blocks
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_0p6b", "bf16_d128_bs32_g2"])
def test_copy_blocks_bit_exact(name):
    """P15 on the GPU: block copies (pairs outside the pool skipped)."""
    inp = inputs_for(name)
    nb = inp["num_blocks"]
    pairs = np.array([[1, nb - 1], [3, 0], [-1, 2], [2, nb], [5, nb - 2], [7, 9]],
                     dtype=np.int64)
    say("copy_blocks", name)
    d = G.upload(inp)
    pa.copy_blocks(d["k_cache"], d["v_cache"], torch.from_numpy(pairs).cuda())
    k_ref, v_ref = oracle.copy_blocks(inp["k_cache"], inp["v_cache"], pairs)
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    assert np.array_equal(G.host_storage(d["v_cache"]), v_ref)


def test_prefix_fork_copy_on_write():
    """Sequences sharing prompt-prefix blocks: sequences 2 and 3 name sequence
    0's first two (full) blocks in their tables; sequence 1 forks sequence 0's
    whole 49-token history, whose last block is partly filled, so it gets a
    private copy of that block before its own new token goes in.  Copy, write
    and decode on the GPU against the oracle taking the same steps."""
    w = synth.Workload("fork_bf16", 4, 8, 2, 128, 16, "bf16", ("uniform", 40, 60),
                       num_blocks=64, seed=41)
    ctx = np.array([50, 50, 45, 58], dtype=np.int32)
    inp = dict(synth.make_inputs(w, context_lens=ctx))
    bs = w.block_size
    tables = inp["block_tables"].copy()
    slots = inp["slot_mapping"].copy()
    last = (int(ctx[0]) - 1) // bs               # block holding position 49
    used = set(int(x) for x in tables[tables >= 0].ravel())
    fresh = next(x for x in range(inp["num_blocks"]) if x not in used)
    tables[1, :] = -1
    tables[1, :last + 1] = tables[0, :last + 1]
    tables[1, last] = fresh
    slots[1] = fresh * bs + (int(ctx[1]) - 1) % bs
    tables[2, :2] = tables[0, :2]
    tables[3, :2] = tables[0, :2]
    pairs = np.array([[tables[0, last], fresh]], dtype=np.int64)
    inp.update(block_tables=tables, slot_mapping=slots)
    say("prefix fork: copy, write, decode")
    d = G.upload(inp)
    pa.copy_blocks(d["k_cache"], d["v_cache"], torch.from_numpy(pairs).cuda())
    out = G.host_f64(gpu_step(d))
    k_ref, v_ref = oracle.copy_blocks(inp["k_cache"], inp["v_cache"], pairs)
    k_ref, v_ref = oracle.reshape_and_cache(inp["key"], inp["value"], k_ref, v_ref, slots)
    ref = oracle.decode(inp["q"], k_ref, v_ref, tables, ctx, inp["scale"], "bf16")
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    assert np.array_equal(G.host_storage(d["v_cache"]), v_ref)
    G.assert_close(out, ref, "bf16", "prefix fork")
    # Sequence 1 saw sequence 0's history, not its new token.
    assert not np.array_equal(out[0], out[1])


# ------------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name,ps,fused,merge", [
    ("qwen3_0p6b", None, False, None), ("mqa_large", None, False, None),
    ("qwen3_0p6b", 64, False, None), ("qwen3_0p6b", None, True, None),
    ("qwen3_0p6b", 64, True, None), ("qwen3_0p6b", None, True, "separate")])
def test_graph_replays_match_eager(name, ps, fused, merge, monkeypatch):
    """A step (KV write + decode, or the fused step) captured in a HIP graph:
    every replay, with eager launches and host synchronisations between
    replays, gives the eager result bit for bit.  The workspace and the
    arrival counters are allocated before capture and passed in, so nothing
    is allocated or cleared inside the graph (the kernels leave the counters
    at zero themselves).  At 64-token partitions the step holds the separate
    merge kernel too, and with merge="separate" the balanced schedule's merge
    kernel."""
    if merge:
        G.setopt(monkeypatch, "PAGEDATTN_MERGE", merge)
    inp = inputs_for(name)
    w = inp["workload"]
    say("graph capture", name, ps, "fused" if fused else "")
    d = G.upload(inp)
    B, hq, hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    mb = d["block_tables"].shape[1]
    ps = w.partition_size if ps is None else ps
    ws = torch.zeros(max(pa.decode_workspace_bytes(B, hq, hkv, w.head_dim, mb, w.block_size,
                                                   ps), 256), dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(B * hkv, dtype=torch.int32, device="cuda")

    def step(out):
        if fused:
            pa.decode_step(d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"],
                           d["block_tables"], d["context_lens"], d["scale"], partition_size=ps,
                           out=out, workspace=ws, counters=cnt)
            return
        pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"],
                             d["slot_mapping"])
        pa.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["context_lens"], d["scale"], partition_size=ps, out=out,
                                  workspace=ws, counters=cnt)

    eager = torch.empty_like(d["q"])
    step(eager)
    torch.cuda.synchronize()
    expect = G.host_storage(eager)
    graphed = torch.full_like(d["q"], float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream
        step(graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graphed)
    scratch = torch.empty_like(d["q"])
    ref, (k_ref, v_ref) = oracle_step(inp)
    for r in range(4):
        graphed.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(G.host_storage(graphed), expect), f"replay {r}"
        # Each replay against the oracle directly (the write is idempotent:
        # every replay writes the same rows to the same slots).
        G.assert_close(G.host_f64(graphed), ref, w.dtype, f"graph replay {r}")
        step(scratch)                    # eager work between replays
        torch.cuda.synchronize()
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    assert np.array_equal(G.host_storage(d["v_cache"]), v_ref)
    assert int(cnt.abs().sum()) == 0


# ------------------------------------------------------------------ prior art
@pytest.mark.parametrize("name", ["qwen3_0p6b", "bf16_d64_bs32_g8"])
def test_prior_art_baseline_matches_oracle(name):
    """The gather-then-attention PyTorch baseline that bench.py times beside
    the kernel computes the same decode (so the comparison is like for like)."""
    import bench
    inp = inputs_for(name)
    w = inp["workload"]
    say("prior-art baseline", name)
    d = G.upload(inp)
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    out, _ = bench.gather_then_attention(d["q"], d["k_cache"], d["v_cache"],
                                         d["block_tables"], d["context_lens"], d["scale"])
    ref, _ = oracle_step(inp)
    G.assert_close(G.host_f64(out), ref, w.dtype, f"{name} baseline")


# ------------------------------------------------------------------ prefill
PF = {
    "pf_g2_d128_bs16": synth.Workload("pf_g2_d128_bs16", 4, 8, 4, 128, 16, "bf16",
                                      ("uniform", 100, 400), seed=51,
                                      query=("uniform", 1, 300)),
    "pf_full_g1_d128_bs32": synth.Workload("pf_full_g1_d128_bs32", 3, 4, 4, 128, 32, "bf16",
                                           ("uniform", 50, 300), seed=52, query=("full",)),
    "pf_g4_d64_bs16": synth.Workload("pf_g4_d64_bs16", 3, 16, 4, 64, 16, "bf16",
                                     ("uniform", 60, 500), seed=53,
                                     query=("uniform", 20, 500)),
    "pf_full_g8_d64_bs32": synth.Workload("pf_full_g8_d64_bs32", 2, 16, 2, 64, 32, "bf16",
                                          ("uniform", 30, 200), seed=54, query=("full",)),
    "pf_g16_d128_bs16": synth.Workload("pf_g16_d128_bs16", 2, 16, 1, 128, 16, "bf16",
                                       ("uniform", 40, 150), seed=55,
                                       query=("uniform", 1, 150)),
    "pf_full_g32_d128_bs32": synth.Workload("pf_full_g32_d128_bs32", 2, 32, 1, 128, 32,
                                            "bf16", ("uniform", 20, 90), seed=56,
                                            query=("full",)),
}


def prefill_gpu(inp):
    """KV write of the new tokens, then prefill, on the GPU."""
    d = G.upload(inp)
    d["query_start"] = torch.from_numpy(inp["query_start"]).cuda()
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    out = pa.paged_attention_prefill(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                     d["context_lens"], d["query_start"], d["scale"])
    return d, out


def prefill_oracle(inp):
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    return oracle.prefill(inp["q"], k, v, inp["block_tables"], inp["context_lens"],
                          inp["query_start"], inp["scale"], inp["workload"].dtype), (k, v)


@pytest.mark.parametrize("ks", ["1", "2"])
@pytest.mark.parametrize("name", list(PF))
def test_prefill_matches_oracle(name, ks, monkeypatch):
    """Every prefill shape, with each wave folding all of its keys (1) and
    with the keys split between two waves per row set (2)."""
    G.setopt(monkeypatch, "PAGEDATTN_PREFILL_KSPLIT", ks)
    w = PF[name]
    inp = synth.make_prefill_inputs(w)
    say("prefill", name, "key halves", ks, "rows",
        int(inp["query_start"][-1]) * (w.num_q_heads // w.num_kv_heads))
    d, out = prefill_gpu(inp)
    ref, (k_ref, _) = prefill_oracle(inp)
    assert np.array_equal(G.host_storage(d["k_cache"]), k_ref)
    G.assert_close(G.host_f64(out), ref, "bf16", name)


@pytest.mark.parametrize("ks", ["1", "2"])
@pytest.mark.parametrize("G_", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_every_shape(D, bs, G_, ks, monkeypatch):
    """Every (head_dim, block size, group) the prefill kernel is built for,
    in both forms, on chunks after cached prefixes (small ragged batch)."""
    G.setopt(monkeypatch, "PAGEDATTN_PREFILL_KSPLIT", ks)
    hkv = 2 if G_ <= 16 else 1
    w = synth.Workload(f"pf_d{D}_bs{bs}_g{G_}", 2, G_ * hkv, hkv, D, bs, "bf16",
                       ("uniform", 40, 300), seed=80 + D + bs + G_, query=("uniform", 1, 200))
    inp = synth.make_prefill_inputs(w)
    say("prefill", w.name, "key halves", ks)
    d, out = prefill_gpu(inp)
    ref, _ = prefill_oracle(inp)
    G.assert_close(G.host_f64(out), ref, "bf16", w.name)


@pytest.mark.parametrize("ks", ["1", "2"])
def test_prefill_ragged_with_empty_and_bad_sequences(ks, monkeypatch):
    """A sequence with no new tokens writes nothing; a sequence claiming more
    new tokens than positions gets NaN rows; the others are unaffected."""
    G.setopt(monkeypatch, "PAGEDATTN_PREFILL_KSPLIT", ks)
    w = PF["pf_g2_d128_bs16"]
    inp = synth.make_prefill_inputs(w, query_lens=np.array([37, 0, 250, 5], dtype=np.int32))
    ctx = inp["context_lens"].copy()
    start = inp["query_start"]
    say("prefill ragged/bad")
    d = G.upload(inp)
    d["query_start"] = torch.from_numpy(start).cuda()
    pa.reshape_and_cache(d["key"], d["value"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    bad = 3
    ctx_bad = ctx.copy()
    ctx_bad[bad] = int(start[bad + 1] - start[bad]) - 1   # fewer positions than new rows
    out = pa.paged_attention_prefill(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                     torch.from_numpy(ctx_bad).cuda(), d["query_start"],
                                     d["scale"])
    got = G.host_f64(out)
    ref, _ = prefill_oracle(inp)
    ok = slice(0, int(start[bad]))
    G.assert_close(got[ok], ref[ok], "bf16", "good sequences")
    assert np.isnan(got[int(start[bad]):int(start[bad + 1])]).all()


def test_prefill_many_sequences():
    """700 sequences (more than a workgroup has threads, so each thread ranks
    several), short prompts and chunks, every seventh sequence with no new
    token: every row of the longest-first schedule is computed once."""
    w = synth.Workload("pf_many", 700, 4, 2, 64, 16, "bf16", ("uniform", 1, 120), seed=57,
                       query=("uniform", 1, 120))
    base = synth.make_prefill_inputs(w)
    qlen = base["query_lens"].copy()
    qlen[::7] = 0
    inp = synth.make_prefill_inputs(w, query_lens=qlen)
    say("prefill 700 sequences, tokens", int(inp["query_start"][-1]))
    _, out = prefill_gpu(inp)
    ref, _ = prefill_oracle(inp)
    G.assert_close(G.host_f64(out), ref, "bf16", "700 sequences")


def test_prefill_wide_cost_buckets():
    """Block tables long enough (262,144 tokens) that the ranking's cost
    buckets are widened to fit its table; the prompts themselves are short."""
    w = synth.Workload("pf_wide", 5, 8, 2, 128, 16, "bf16", ("uniform", 50, 700), seed=58,
                       query=("uniform", 1, 700), max_blocks=16384)
    inp = synth.make_prefill_inputs(w)
    say("prefill wide buckets, tokens", int(inp["query_start"][-1]))
    _, out = prefill_gpu(inp)
    ref, _ = prefill_oracle(inp)
    G.assert_close(G.host_f64(out), ref, "bf16", "wide buckets")


@pytest.mark.parametrize("name", ["pf_g2_d128_bs16", "pf_full_g32_d128_bs32",
                                  "pf_g4_d64_bs16"])
def test_prefill_first_token_exact(name):
    """P20 on the GPU: a one-token prompt returns exactly its own V row."""
    w = PF[name]
    one = np.ones(w.num_seqs, dtype=np.int32)
    inp = synth.make_prefill_inputs(w, context_lens=one, query_lens=one)
    say("prefill one-token prompts", name)
    _, out = prefill_gpu(inp)
    got = G.host_storage(out)
    grp = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        assert np.array_equal(got[b], np.repeat(inp["value"][b], grp, axis=0)), b


@pytest.mark.parametrize("name", list(synth.PREFILL_WORKLOADS))
def test_prefill_workload_sampled(name):
    """The benchmark prefill batches at full size: every row of every sequence
    is computed on the GPU; sampled rows are checked one by one against the
    oracle's decode ending at the row's position (P17)."""
    w = synth.PREFILL_WORKLOADS[name]
    inp = synth.make_prefill_inputs(w)
    say("prefill workload", name, "tokens", int(inp["query_start"][-1]))
    d, out = prefill_gpu(inp)
    got = G.host_f64(out)
    assert np.isfinite(got).all()
    k, v = oracle.reshape_and_cache(inp["key"], inp["value"], inp["k_cache"],
                                    inp["v_cache"], inp["slot_mapping"])
    rng = np.random.default_rng(9)
    ctx, start = inp["context_lens"], inp["query_start"]
    for b in range(w.num_seqs):
        n = int(start[b + 1] - start[b])
        for i in sorted(set(rng.integers(0, n, size=6).tolist()) | {0, n - 1}):
            row = int(start[b]) + i
            pos = int(ctx[b]) - n + i
            ref = oracle.decode(inp["q"][row:row + 1], k, v, inp["block_tables"][b:b + 1],
                                np.array([pos + 1], dtype=np.int32), inp["scale"], w.dtype)
            G.assert_close(got[row:row + 1], ref, w.dtype, f"{name} seq {b} row {i}")
