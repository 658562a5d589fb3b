"""Plain float64 definitions of the paged KV write and paged decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow on purpose, written so
that each step can be checked against the pages by eye.  All pins live in
``tests/test_oracle_pins.py``; every function here is pinned there by something
other than itself (closed forms, invariants, a library routine, 50-digit brute
force).

What the pages fix, and where:
  * Storage is one ``[num_blocks, block_size, kv_heads, head_dim]`` K tensor and
    one V tensor per layer, token before head (barellm README: the paged-cache
    component list names the ``[layers, physical_blocks, block_size, kv_heads,
    head_dim]`` tensors; its feature list states the token-before-head order).
  * A position is found through the request's block table: logical block
    ``pos // block_size``, looked up to a physical block (barellm README, the
    address-mapping line at the end of the paged-cache list).  The offset inside
    the block, ``pos % block_size``, is the plain reading of that line.
  * The cache owns the logical-to-physical *writes* (barellm README, paged-cache
    component list) -- this is ``reshape_and_cache``.
  * Paged attention computes the same attention as a contiguous cache: barellm
    gathers pages into dense tensors and runs ordinary attention, and tests
    paged against contiguous storage for MHA, GQA and MQA (barellm README,
    feature list).  So decode is softmax attention of one query over the first
    ``context_lens[b]`` cached tokens of sequence b, after an exact gather.
  * Grouped heads: several query heads share one KV head (barellm feature list:
    GQA/MQA; CUDAlab README, Benchmark: the ``kv_mul`` flag; LLAISYS README,
    self-attention item: GQA by broadcasting).  Reading taken: query head h uses
    KV head ``h // (Hq // Hkv)``, i.e. contiguous groups.
  * The score is ``scale * q . k``; softmax subtracts the running maximum and
    sums ``exp``; the output is the weighted sum of V divided by that sum
    (LLAISYS README, self-attention item: online softmax with running max and
    running sum; MinivLLM article, "What the Two Benchmark Scripts Compare":
    blockwise online softmax).

Readings where the pages are silent: ``context_lens`` counts the token written
this step; a slot is ``physical_block * block_size + offset`` and a negative
slot writes nothing; a sequence of length 0 yields a zero output row.
"""
from __future__ import annotations

import numpy as np


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.

    ``dtype == "bf16"``: ``x`` holds bfloat16 bit patterns (uint16); a bfloat16
    is the upper half of a float32, so shifting the bits up by 16 gives the same
    number as a float32, which float64 then holds exactly.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """The paged KV write.  Returns new (k_cache, v_cache); inputs untouched.

    For each new token i with ``slot = slot_mapping[i] >= 0``: the row
    ``key[i]`` (all KV heads, all dims) goes to physical block
    ``slot // block_size`` at offset ``slot % block_size``; the same for
    ``value``.  A pure copy of the stored bits.  Duplicate slots within one
    call are outside the contract.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    block_size = k_cache.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = slot // block_size, slot % block_size
        k_out[blk, off] = key[i]
        v_out[blk, off] = value[i]
    return k_out, v_out


def copy_blocks(k_cache, v_cache, block_pairs):
    """Copy-on-write of shared blocks.  Returns new (k_cache, v_cache).

    Sequences with a common prompt prefix may name the same physical blocks
    in their tables (block sharing: MinivLLM article, "Running It" section;
    prefix caching: nano-vllm overview, "Kernmodul: Sequence").  Reading
    taken where the pages are silent: before one of them writes into a shared
    block it gets a private copy.  For each (src, dst) row of ``block_pairs``,
    in order, with both ids inside the pool: block dst of both caches becomes
    a copy of block src.  Rows naming a block outside the pool are skipped.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_blocks = k_cache.shape[0]
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks):
            continue
        k_out[dst] = k_out[src]
        v_out[dst] = v_out[src]
    return k_out, v_out


def gather_kv(cache, block_tables, context_lens):
    """Exact gather of each sequence's cached rows into a dense tensor.

    Returns ``[B, max_blocks * block_size, kv_heads, head_dim]`` in the storage
    dtype: row t of sequence b is ``cache[block_tables[b, t // bs], t % bs]``
    for ``t < context_lens[b]`` and zero after it.  Table entries at or past
    ``ceil(ctx / bs)`` are never looked at.
    """
    B, max_blocks = block_tables.shape
    bs = cache.shape[1]
    out = np.zeros((B, max_blocks * bs) + cache.shape[2:], dtype=cache.dtype)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        pos = np.arange(L)
        phys = block_tables[b, pos // bs].astype(np.int64)
        out[b, :L] = cache[phys, pos % bs]
    return out


def decode_one(q_b, K, V, scale):
    """Softmax attention of one sequence's query heads over dense K/V rows.

    ``q_b``: [Hq, D] float64; ``K``, ``V``: [L, Hkv, D] float64.  Query head h
    reads KV head ``h // (Hq // Hkv)``.  Returns [Hq, D] float64 (zeros if L == 0).
    """
    Hq, D = q_b.shape
    L, Hkv, _ = K.shape
    if L == 0:
        return np.zeros((Hq, D))
    group = Hq // Hkv
    kv_head = np.arange(Hq) // group
    Kh = K[:, kv_head, :]  # [L, Hq, D]
    Vh = V[:, kv_head, :]
    s = np.float64(scale) * np.einsum("hd,thd->ht", q_b, Kh)  # [Hq, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    num = np.einsum("ht,thd->hd", p, Vh)
    return num / p.sum(axis=1)[:, None]


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Paged decode attention, float64.  Returns out [B, Hq, D] (float64).

    ``scale`` is taken as the float32 value the library receives, widened.
    """
    scale = np.float64(np.float32(scale))
    qf = widen(q, dtype)
    B = qf.shape[0]
    bs = k_cache.shape[1]
    out = np.zeros(qf.shape, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        pos = np.arange(L)
        phys = block_tables[b, pos // bs].astype(np.int64)
        K = widen(k_cache[phys, pos % bs], dtype)
        V = widen(v_cache[phys, pos % bs], dtype)
        out[b] = decode_one(qf[b], K, V, scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype):
    """Paged prefill (and chunked-prefill) attention, causal, float64.

    The step before decode on the pages' data flow: a prompt, or a chunk of
    it after a cached prefix, is processed at once, each new token attending
    to every cached position up to its own (MinivLLM article, "Engine
    Layout": prefilling vs decoding; nano-vllm overview, "Prefill vs.
    Decode").  Sequence b's new query rows are
    ``q[query_start[b] : query_start[b+1]]``; with ``L = context_lens[b]`` and
    ``n`` new rows, row i sits at position ``L - n + i`` and attends to the
    cached positions ``0 .. L - n + i`` (its own row, written by the KV write,
    included).  Returns out [T, Hq, D] float64; rows of a sequence with
    ``n > L`` are NaN (there is no such position).
    """
    scale = np.float64(np.float32(scale))
    qf = widen(q, dtype)
    out = np.zeros(qf.shape, dtype=np.float64)
    bs = k_cache.shape[1]
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        lo, hi = int(query_start[b]), int(query_start[b + 1])
        n = hi - lo
        if n <= 0:
            continue
        if n > L:
            out[lo:hi] = np.nan
            continue
        pos = np.arange(L)
        phys = block_tables[b, pos // bs].astype(np.int64)
        K = widen(k_cache[phys, pos % bs], dtype)
        V = widen(v_cache[phys, pos % bs], dtype)
        for i in range(n):
            p = L - n + i
            out[lo + i] = decode_one(qf[lo + i], K[:p + 1], V[:p + 1], scale)
    return out


def decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                    dtype, partition_size):
    """Per-partition softmax state, for the split-K merge identity.

    The tokens of each sequence are cut into consecutive partitions of
    ``partition_size`` positions.  For each (b, h, partition): ``m`` the maximum
    score, ``l = sum exp(s - m)``, ``acc = sum exp(s - m) v`` (unnormalised).
    Empty partitions have m = -inf, l = 0, acc = 0.  Returns (m, l, acc) with
    shapes [B, Hq, P], [B, Hq, P], [B, Hq, P, D].
    """
    scale = np.float64(np.float32(scale))
    qf = widen(q, dtype)
    B, Hq, D = qf.shape
    bs = k_cache.shape[1]
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    kv_head = np.arange(Hq) // group
    P = max(1, -(-int(np.max(context_lens)) // partition_size))
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    acc = np.zeros((B, Hq, P, D))
    for b in range(B):
        L = int(context_lens[b])
        for p in range(P):
            lo, hi = p * partition_size, min(L, (p + 1) * partition_size)
            if hi <= lo:
                continue
            pos = np.arange(lo, hi)
            phys = block_tables[b, pos // bs].astype(np.int64)
            K = widen(k_cache[phys, pos % bs], dtype)[:, kv_head, :]
            V = widen(v_cache[phys, pos % bs], dtype)[:, kv_head, :]
            s = scale * np.einsum("hd,thd->ht", qf[b], K)
            mp = s.max(axis=1)
            e = np.exp(s - mp[:, None])
            m[b, :, p] = mp
            l[b, :, p] = e.sum(axis=1)
            acc[b, :, p] = np.einsum("ht,thd->hd", e, V)
    return m, l, acc


def merge_partials(m, l, acc):
    """Log-sum-exp merge of partition states into the attention output.

    M = max_p m_p;  L = sum_p l_p exp(m_p - M);  out = sum_p acc_p exp(m_p - M) / L.
    Rows whose partitions are all empty give zeros.
    """
    B, Hq, P = m.shape
    out = np.zeros(acc.shape[:2] + acc.shape[3:])
    for b in range(B):
        for h in range(Hq):
            valid = np.isfinite(m[b, h])
            if not valid.any():
                continue
            M = m[b, h, valid].max()
            w = np.exp(m[b, h, valid] - M)
            Lsum = (l[b, h, valid] * w).sum()
            out[b, h] = (acc[b, h, valid] * w[:, None]).sum(axis=0) / Lsum
    return out
