"""Seeded synthetic inputs for paged decode attention and the paged KV write.

This module only *builds inputs*: context lengths, a physical block pool, block
tables, query / key / value tensors and the slot of each sequence's newest token.
It holds none of the attention arithmetic.  Both the CPU oracle (through the
tests) and the HIP path consume exactly the arrays made here.

Workload shapes follow the pages' model families and cache layout:
  * paged storage is ``[num_blocks, block_size, kv_heads, head_dim]`` per layer,
    token before head (barellm README, paged-cache component list and the NHD
    layout note in its feature list);
  * each request owns a block table mapping logical block ``pos // block_size``
    to a physical block (barellm README, paged-cache component list);
  * Qwen3-0.6B-like and Llama-3.2-1B-like head shapes (nano-vllm overview,
    "Leistungsbenchmark und Ergebnisse"; CUDAlab README, 批量推理 / Benchmark).

Storage dtypes: ``"f32"`` arrays are ``np.float32``; ``"bf16"`` arrays are
``np.uint16`` holding bfloat16 bit patterns (numpy has no bfloat16), produced by
round-to-nearest-even from float32 draws.

Readings taken where the pages are silent (all listed in the design notes):
  * ``context_lens[b]`` counts the token being written this step, which sits at
    position ``context_lens[b] - 1``;
  * a slot is ``physical_block * block_size + offset``; a negative slot means
    "write nothing";
  * padded block-table entries are ``-1`` (or, in poison runs, the id of a
    NaN-filled spare block);
  * physical blocks are handed out from one seeded permutation of the pool, in
    batch order; the pool holds ``max(ceil(1.25 * sum(ctx) / bs), sum(ceil(ctx / bs)))``
    blocks unless the workload fixes it;
  * ``uniform in [a, b]`` is an inclusive integer draw.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "PREFILL_WORKLOADS",
    "make_prefill_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "storage_np_dtype",
]


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one decode batch (one attention layer)."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" | "bf16"
    ctx: tuple  # ("fixed", (c0, c1, ...)) | ("uniform", lo, hi) | ("const", c)
    sigma: float = 1.0
    num_blocks: int | None = None  # None: pool rule (1.25 x total tokens)
    max_blocks: int | None = None  # None: ceil(largest possible ctx / block_size)
    partition_size: int = 0  # 0: library chooses
    seed: int = 0
    # Prefill only: new query tokens per sequence, the last ones of its
    # context.  ("full",): the whole context (a prompt from scratch);
    # ("uniform", lo, hi) / ("fixed", (n0, n1, ...)): a chunk after a cached
    # prefix, clipped to the context length.
    query: tuple | None = None

    @property
    def max_ctx(self) -> int:
        kind = self.ctx[0]
        if kind == "fixed":
            return max(self.ctx[1])
        if kind == "uniform":
            return self.ctx[2]
        return self.ctx[1]

    @property
    def max_blocks_per_seq(self) -> int:
        if self.max_blocks is not None:
            return self.max_blocks
        return max(1, -(-self.max_ctx // self.block_size))

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five decode workloads, plus the MQA rerun of the large-batch one.
WORKLOADS: dict[str, Workload] = {
    "tiny_f32": Workload(
        "tiny_f32", 4, 4, 2, 64, 16, "f32", ("fixed", (1, 17, 33, 64)),
        num_blocks=32, max_blocks=4, seed=1001),
    "qwen3_0p6b": Workload(
        "qwen3_0p6b", 32, 16, 8, 128, 16, "bf16", ("uniform", 128, 2048),
        max_blocks=128, seed=1002),
    "llama32_1b": Workload(
        "llama32_1b", 64, 32, 8, 64, 16, "bf16", ("uniform", 1, 4096),
        max_blocks=256, seed=1003),
    "long_splitk": Workload(
        "long_splitk", 8, 32, 8, 128, 16, "bf16", ("const", 32768),
        max_blocks=2048, partition_size=512, seed=1004),
    "mha_large": Workload(
        "mha_large", 256, 32, 32, 128, 32, "bf16", ("uniform", 1, 1024),
        sigma=0.5, max_blocks=32, seed=1005),
    "mqa_large": Workload(
        "mqa_large", 256, 32, 1, 128, 32, "bf16", ("uniform", 1, 1024),
        sigma=0.5, max_blocks=32, seed=1005),
}


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    NaN stays a quiet NaN.  Input generation only (values handed to both sides).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str,
          chunk: int = 1 << 24) -> np.ndarray:
    """N(0, sigma) draws in float32, stored in the workload dtype.

    Drawn in fixed-size chunks so multi-GB pools never need a float32 copy of
    the whole pool; chunking is part of the recipe, so results are reproducible.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=storage_np_dtype(dtype))
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        out[s:e] = v if dtype == "f32" else f32_to_bf16_bits(v)
    return out.reshape(shape)


def _nan_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)


def draw_context_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.ctx[0]
    if kind == "fixed":
        vals = np.asarray(w.ctx[1], dtype=np.int64)
        assert vals.size == w.num_seqs
    elif kind == "uniform":
        vals = rng.integers(w.ctx[1], w.ctx[2], size=w.num_seqs, endpoint=True)
    elif kind == "const":
        vals = np.full(w.num_seqs, w.ctx[1], dtype=np.int64)
    else:
        raise ValueError(kind)
    return vals.astype(np.int32)


def pool_blocks(w: Workload, ctx: np.ndarray) -> int:
    used = int(sum(-(-int(c) // w.block_size) for c in ctx))
    if w.num_blocks is not None:
        if w.num_blocks < used:
            raise ValueError("pool too small for the context lengths")
        return w.num_blocks
    return max(math.ceil(1.25 * int(ctx.sum()) / w.block_size), used)


def make_inputs(w: Workload, seed: int | None = None, poison: bool = False,
                context_lens=None) -> dict:
    """Build one decode batch.

    Generation order: context lengths -> block permutation -> K pool -> V pool
    -> q -> new key / value rows.  ``context_lens`` overrides the drawn lengths
    (the generator still draws them, so every later array is unchanged).

    With ``poison=True`` the arrays are identical except that every cache slot
    that no sequence may read (unused blocks, slots past each sequence's length
    in its last block) holds NaN, and padded block-table entries point at a
    NaN-filled spare block instead of -1.

    Returns a dict with numpy arrays: ``context_lens`` int32 [B],
    ``block_tables`` int32 [B, max_blocks], ``k_cache``/``v_cache``
    [num_blocks, bs, Hkv, D], ``q`` [B, Hq, D], ``key``/``value`` [B, Hkv, D],
    ``slot_mapping`` int64 [B] (slot of position ctx-1, or -1 when ctx == 0),
    ``scale`` (np.float32, 1/sqrt(D)) and the scalar sizes.
    """
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, bs = (w.num_seqs, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, w.block_size)
    ctx = draw_context_lens(w, rng)
    if context_lens is not None:
        ctx = np.asarray(context_lens, dtype=np.int32).copy()
        assert ctx.shape == (B,)
    max_blocks = w.max_blocks_per_seq
    nblk = [-(-int(c) // bs) for c in ctx]
    if max(nblk) > max_blocks:
        raise ValueError("context longer than max_blocks * block_size")
    num_blocks = pool_blocks(w, ctx)
    perm = rng.permutation(num_blocks).astype(np.int32)

    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[cursor:cursor + nblk[b]]
        cursor += nblk[b]
    unused = perm[cursor:]

    k_cache = _draw(rng, (num_blocks, bs, Hkv, D), w.sigma, w.dtype)
    v_cache = _draw(rng, (num_blocks, bs, Hkv, D), w.sigma, w.dtype)
    q = _draw(rng, (B, Hq, D), w.sigma, w.dtype)
    key = _draw(rng, (B, Hkv, D), w.sigma, w.dtype)
    value = _draw(rng, (B, Hkv, D), w.sigma, w.dtype)

    slots = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        c = int(ctx[b])
        if c > 0:
            pos = c - 1
            slots[b] = int(tables[b, pos // bs]) * bs + pos % bs

    if poison:
        if unused.size == 0:
            raise ValueError("poison run needs a spare block")
        nanv = _nan_value(w.dtype)
        k_cache[unused] = nanv
        v_cache[unused] = nanv
        for b in range(B):
            c = int(ctx[b])
            if c % bs:
                last = tables[b, nblk[b] - 1]
                k_cache[last, c % bs:] = nanv
                v_cache[last, c % bs:] = nanv
        tables[tables < 0] = unused[0]

    return dict(
        workload=w, seed=seed, context_lens=ctx, block_tables=tables,
        num_blocks=num_blocks, k_cache=k_cache, v_cache=v_cache, q=q,
        key=key, value=value, slot_mapping=slots,
        scale=np.float32(1.0 / math.sqrt(D)), max_blocks=max_blocks,
    )


# Prefill (and chunked-prefill) batches: several query tokens per sequence,
# causal over the sequence's cached positions.
PREFILL_WORKLOADS: dict[str, Workload] = {
    "prefill_qwen3": Workload(
        "prefill_qwen3", 8, 16, 8, 128, 16, "bf16", ("uniform", 512, 2048),
        max_blocks=128, seed=1101, query=("full",)),
    "chunked_qwen3": Workload(
        "chunked_qwen3", 8, 16, 8, 128, 16, "bf16", ("uniform", 1024, 4096),
        max_blocks=256, seed=1102, query=("uniform", 128, 512)),
    "prefill_llama32_1b": Workload(
        "prefill_llama32_1b", 8, 32, 8, 64, 16, "bf16", ("uniform", 256, 2048),
        max_blocks=128, seed=1103, query=("full",)),
}


def draw_query_lens(w: Workload, ctx: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    kind = w.query[0]
    if kind == "full":
        n = ctx.astype(np.int64)
    elif kind == "uniform":
        n = rng.integers(w.query[1], w.query[2], size=w.num_seqs, endpoint=True)
    elif kind == "fixed":
        n = np.asarray(w.query[1], dtype=np.int64)
        assert n.size == w.num_seqs
    else:
        raise ValueError(kind)
    return np.minimum(n, ctx).astype(np.int32)


def make_prefill_inputs(w: Workload, seed: int | None = None, context_lens=None,
                        query_lens=None) -> dict:
    """Build one prefill (or chunked-prefill) batch.

    Generation order: context lengths -> query lengths -> block permutation ->
    K pool -> V pool -> q -> new key / value rows.  Sequence b brings
    ``query_lens[b]`` new tokens, the last ones of its ``context_lens[b]``
    positions; the positions before them (a cached prefix, possibly empty)
    hold whatever the pool holds.

    Returns numpy arrays: ``context_lens`` int32 [B], ``query_lens`` int32 [B],
    ``query_start`` int32 [B+1] (sequence b's rows of q are
    query_start[b] .. query_start[b+1]-1), ``block_tables`` int32
    [B, max_blocks], ``k_cache``/``v_cache`` [num_blocks, bs, Hkv, D], ``q``
    [T, Hq, D], ``key``/``value`` [T, Hkv, D] (the new tokens' rows),
    ``slot_mapping`` int64 [T] (each new token's slot), ``scale`` and sizes.
    """
    assert w.query is not None, "not a prefill workload"
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, bs = (w.num_seqs, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, w.block_size)
    ctx = draw_context_lens(w, rng)
    if context_lens is not None:
        ctx = np.asarray(context_lens, dtype=np.int32).copy()
    qlen = draw_query_lens(w, ctx, rng)
    if query_lens is not None:
        qlen = np.minimum(np.asarray(query_lens, dtype=np.int32), ctx)
    max_blocks = w.max_blocks_per_seq
    nblk = [-(-int(c) // bs) for c in ctx]
    if max(nblk) > max_blocks:
        raise ValueError("context longer than max_blocks * block_size")
    num_blocks = pool_blocks(w, ctx)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[cursor:cursor + nblk[b]]
        cursor += nblk[b]

    T = int(qlen.sum())
    k_cache = _draw(rng, (num_blocks, bs, Hkv, D), w.sigma, w.dtype)
    v_cache = _draw(rng, (num_blocks, bs, Hkv, D), w.sigma, w.dtype)
    q = _draw(rng, (T, Hq, D), w.sigma, w.dtype)
    key = _draw(rng, (T, Hkv, D), w.sigma, w.dtype)
    value = _draw(rng, (T, Hkv, D), w.sigma, w.dtype)

    start = np.zeros(B + 1, dtype=np.int32)
    start[1:] = np.cumsum(qlen)
    slots = np.empty(T, dtype=np.int64)
    for b in range(B):
        first = int(ctx[b]) - int(qlen[b])
        for i in range(int(qlen[b])):
            pos = first + i
            slots[start[b] + i] = int(tables[b, pos // bs]) * bs + pos % bs

    return dict(
        workload=w, seed=seed, context_lens=ctx, query_lens=qlen, query_start=start,
        block_tables=tables, num_blocks=num_blocks, k_cache=k_cache, v_cache=v_cache,
        q=q, key=key, value=value, slot_mapping=slots,
        scale=np.float32(1.0 / math.sqrt(D)), max_blocks=max_blocks,
        max_query_len=int(qlen.max()) if B else 0,
    )
