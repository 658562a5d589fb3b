"""Pins of the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes the oracle functions it exercises as arguments (so the
mutation tests can hand it deliberately broken copies) and returns
``(ok, detail)``.  Sources of truth used here, none of them the oracle itself:
closed forms (a single token, a zero scale, a hard maximum), invariants the
pages state (paged == contiguous storage, GQA/MQA == MHA with replicated KV
heads, uncached recompute == cached decode), a library routine (PyTorch's
``scaled_dot_product_attention`` on the CPU in float64) and 50-digit brute
force with mpmath.
"""
from __future__ import annotations

import math

import numpy as np

import synth


def _np(x):
    return np.asarray(x)


# ---------------------------------------------------------------- helpers
def widen_ref(x, dtype):
    """Independent widening through torch's own bfloat16 type."""
    import torch
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def dense_from_chunks(cache, table_row, L):
    """Rebuild one sequence's dense rows by walking its blocks in order.

    Paging cuts a sequence into consecutive chunks of ``block_size`` tokens and
    stores chunk j in physical block ``table_row[j]`` (rows 0..len-1).  This is
    that statement read backwards, written without any divmod on positions.
    """
    bs = cache.shape[1]
    rows = []
    j = 0
    remaining = L
    while remaining > 0:
        take = min(bs, remaining)
        rows.append(cache[int(table_row[j]), :take])
        remaining -= take
        j += 1
    if not rows:
        return cache[:0, 0]
    return np.concatenate(rows, axis=0)


def sdpa_ref(q_b, K, V, scale):
    """torch SDPA (CPU, float64) over dense rows, KV heads repeated per group."""
    import torch
    Hq, D = q_b.shape
    L, Hkv, _ = K.shape
    rep = Hq // Hkv
    qt = torch.from_numpy(q_b).reshape(1, Hq, 1, D)
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(rep, dim=0).unsqueeze(0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(rep, dim=0).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), scale=float(scale))
    return o.reshape(Hq, D).numpy()


def written(inp, rac):
    """Caches after the step's write of the new token rows."""
    return rac(inp["key"], inp["value"], inp["k_cache"], inp["v_cache"],
               inp["slot_mapping"])


# ---------------------------------------------------------------- KV write
def pin_write_slots(rac, inp):
    """P1: written slots hold the new rows bit for bit; all other slots keep
    their old bits; negative slots write nothing.

    Expected values use the flat-slot view of the cache: a
    ``[num_blocks, bs, ...]`` array seen as ``[num_blocks * bs, ...]`` has
    slot ``blk * bs + off`` at flat row ``slot`` -- row-major layout, no divmod.
    """
    kc, vc = inp["k_cache"], inp["v_cache"]
    slots = np.asarray(inp["slot_mapping"], dtype=np.int64)
    k2, v2 = rac(inp["key"], inp["value"], kc, vc, slots)
    nb, bs = kc.shape[:2]
    flat_k_old = kc.reshape((nb * bs,) + kc.shape[2:])
    flat_v_old = vc.reshape((nb * bs,) + vc.shape[2:])
    flat_k = k2.reshape((nb * bs,) + kc.shape[2:])
    flat_v = v2.reshape((nb * bs,) + vc.shape[2:])
    touched = np.zeros(nb * bs, dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        touched[s] = True
        if flat_k[s].tobytes() != _np(inp["key"][i]).tobytes():
            return False, f"key row {i} not at slot {s}"
        if flat_v[s].tobytes() != _np(inp["value"][i]).tobytes():
            return False, f"value row {i} not at slot {s}"
    if flat_k[~touched].tobytes() != flat_k_old[~touched].tobytes():
        return False, "an untouched K slot changed"
    if flat_v[~touched].tobytes() != flat_v_old[~touched].tobytes():
        return False, "an untouched V slot changed"
    return True, ""


# ---------------------------------------------------------------- gather
def pin_gather_chunks(gather, inp):
    """P2: the gather equals the chunk-by-chunk rebuild, zero past ctx, bitwise."""
    tables, ctx = inp["block_tables"], inp["context_lens"]
    for cache in (inp["k_cache"], inp["v_cache"]):
        g = gather(cache, tables, ctx)
        for b in range(len(ctx)):
            L = int(ctx[b])
            ref = dense_from_chunks(cache, tables[b], L)
            if g[b, :L].tobytes() != ref.tobytes():
                return False, f"seq {b}: rows differ"
            if np.any(g[b, L:].view(np.uint8)):
                return False, f"seq {b}: non-zero padding"
    return True, ""


# ---------------------------------------------------------------- decode
def _dec(dec, inp, k, v, **over):
    args = dict(q=inp["q"], k_cache=k, v_cache=v,
                block_tables=inp["block_tables"],
                context_lens=inp["context_lens"], scale=inp["scale"],
                dtype=inp["workload"].dtype)
    args.update(over)
    return dec(args["q"], args["k_cache"], args["v_cache"], args["block_tables"],
               args["context_lens"], args["scale"], args["dtype"])


def pin_single_token(dec, rac, w):
    """P3: with one cached token, softmax of one score is exactly 1, so the
    output is exactly that token's V row."""
    inp = synth.make_inputs(w, context_lens=np.ones(w.num_seqs, dtype=np.int32))
    k, v = written(inp, rac)
    out = _dec(dec, inp, k, v)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        blk = int(inp["block_tables"][b, 0])
        vrow = widen_ref(v[blk, 0], w.dtype)  # [Hkv, D]
        for h in range(w.num_q_heads):
            if not np.array_equal(out[b, h], vrow[h // G]):
                return False, f"b={b} h={h}"
    return True, ""


def onehot_inputs(w, start_seed=7000, gap=1e-2):
    """Inputs whose top-two raw q.k scores differ by >= gap for every (b, h).

    Raw scores are computed here by plain per-token dot products (no oracle).
    Returns (inputs, caches after the write, expected argmax rows).
    """
    from oracle import reshape_and_cache as _rac  # the write is pinned by P1
    G = w.num_q_heads // w.num_kv_heads
    for seed in range(start_seed, start_seed + 200):
        inp = synth.make_inputs(w, seed=seed)
        k, v = _rac(inp["key"], inp["value"], inp["k_cache"], inp["v_cache"],
                    inp["slot_mapping"])
        q = widen_ref(inp["q"], w.dtype)
        ok = True
        best = {}
        for b in range(w.num_seqs):
            L = int(inp["context_lens"][b])
            dense_k = widen_ref(dense_from_chunks(k, inp["block_tables"][b], L), w.dtype)
            dense_v = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
            for h in range(w.num_q_heads):
                raw = np.array([float(np.dot(q[b, h], dense_k[t, h // G]))
                                for t in range(L)])
                order = np.argsort(raw)
                if L >= 2 and raw[order[-1]] - raw[order[-2]] < gap:
                    ok = False
                    break
                best[(b, h)] = dense_v[order[-1], h // G]
            if not ok:
                break
        if ok:
            return inp, (k, v), best
    raise RuntimeError("no seed with a clear maximum")


def pin_onehot(dec, w):
    """P4: with scale 1e5 every non-maximal weight underflows to exactly 0 and
    the maximal one is exp(0) = 1, so the output is exactly V[argmax]."""
    inp, (k, v), best = onehot_inputs(w)
    out = _dec(dec, inp, k, v, scale=np.float32(1e5))
    for (b, h), row in best.items():
        if not np.array_equal(out[b, h], row):
            return False, f"b={b} h={h}"
    return True, ""


def pin_block_permutation(dec, rac, w, seed=11):
    """P5: relabelling physical blocks (table updated to match) changes nothing."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    base = _dec(dec, inp, k, v)
    rng = np.random.default_rng(seed)
    nb = k.shape[0]
    perm = rng.permutation(nb)  # old block id -> new block id
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    t = inp["block_tables"]
    t2 = np.where(t >= 0, perm[np.clip(t, 0, None)], t).astype(np.int32)
    out = _dec(dec, inp, k2, v2, block_tables=t2)
    if not np.array_equal(out, base):
        return False, f"max diff {np.max(np.abs(out - base))}"
    return True, ""


def pin_gqa_equals_mha(dec, rac, w):
    """P6: grouped heads == MHA over a cache whose KV heads are repeated
    (each KV head copied G times, adjacent), the pages' MHA/GQA/MQA
    equivalence."""
    G = w.num_q_heads // w.num_kv_heads
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    base = _dec(dec, inp, k, v)
    k_rep = np.repeat(k, G, axis=2)
    v_rep = np.repeat(v, G, axis=2)
    out = _dec(dec, inp, k_rep, v_rep)
    if not np.array_equal(out, base):
        return False, f"max diff {np.max(np.abs(out - base))}"
    return True, ""


def pin_split_merge(dec, decode_partials, merge_partials, rac, w, partition_size):
    """P7: splitting positions into partitions and merging with log-sum-exp
    equals the one-pass result (an exact identity; fp64 rounding only)."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    base = _dec(dec, inp, k, v)
    m, l, acc = decode_partials(inp["q"], k, v, inp["block_tables"],
                                inp["context_lens"], inp["scale"],
                                w.dtype, partition_size)
    out = merge_partials(m, l, acc)
    err = np.max(np.abs(out - base))
    # a partition split in the wrong place would leave tokens out
    return (err <= 1e-12), f"max diff {err}"


def pin_contiguous(dec, rac, w):
    """P8: the same rows stored contiguously ([B, Lmax, Hkv, D], i.e. one
    block per sequence and the identity table) give the same output."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    base = _dec(dec, inp, k, v)
    ctx = inp["context_lens"]
    B = len(ctx)
    Lmax = int(ctx.max())
    kc = np.zeros((B, Lmax) + k.shape[2:], dtype=k.dtype)
    vc = np.zeros_like(kc)
    for b in range(B):
        L = int(ctx[b])
        kc[b, :L] = dense_from_chunks(k, inp["block_tables"][b], L)
        vc[b, :L] = dense_from_chunks(v, inp["block_tables"][b], L)
    table = np.arange(B, dtype=np.int32)[:, None]
    out = _dec(dec, inp, kc, vc, block_tables=table)
    if not np.array_equal(out, base):
        return False, f"max diff {np.max(np.abs(out - base))}"
    return True, ""


def pin_uncached_recompute(dec, rac, Hq=4, Hkv=2, D=16, T=40, bs=4, seed=3):
    """P9: decoding step by step from the paged cache (write the token, then
    attend) equals full causal attention over the whole sequence, recomputed
    from scratch with torch SDPA (is_causal) -- the pages' uncached reference."""
    import torch
    rng = np.random.default_rng(seed)
    nblk = -(-T // bs) + 3
    perm = rng.permutation(nblk).astype(np.int32)
    table = perm[: -(-T // bs)][None, :]
    Q = rng.standard_normal((T, Hq, D))
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    Qf = Q.astype(np.float32)
    Kf = K.astype(np.float32)
    Vf = V.astype(np.float32)
    kc = np.zeros((nblk, bs, Hkv, D), dtype=np.float32)
    vc = np.zeros_like(kc)
    scale = np.float32(1 / math.sqrt(D))
    outs = []
    for t in range(T):
        slot = np.array([table[0, t // bs] * bs + t % bs], dtype=np.int64)
        kc, vc = rac(Kf[t:t + 1], Vf[t:t + 1], kc, vc, slot)
        o = dec(Qf[t:t + 1], kc, vc, table, np.array([t + 1], dtype=np.int32),
                scale, "f32")
        outs.append(o[0])
    got = np.stack(outs)  # [T, Hq, D]
    G = Hq // Hkv
    qt = torch.from_numpy(Qf.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(Kf.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0)
    vt = torch.from_numpy(Vf.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), is_causal=True,
        scale=float(scale))[0].permute(1, 0, 2).numpy()
    err = np.max(np.abs(got - ref))
    return err <= 1e-12, f"max diff {err}"


def pin_sdpa(dec, rac, w):
    """P10: PyTorch SDPA (CPU, float64) over the chunk-rebuilt dense rows."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    out = _dec(dec, inp, k, v)
    q = widen_ref(inp["q"], w.dtype)
    worst = 0.0
    for b in range(w.num_seqs):
        L = int(inp["context_lens"][b])
        K = widen_ref(dense_from_chunks(k, inp["block_tables"][b], L), w.dtype)
        V = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
        ref = sdpa_ref(q[b], K, V, np.float64(inp["scale"]))
        worst = max(worst, float(np.max(np.abs(out[b] - ref))))
    return worst <= 1e-12, f"max diff {worst}"


def pin_mpmath(dec, rac, w, digits=50):
    """P11: brute force at 50 significant digits (exp, sums and division in
    mpmath) agrees with the float64 oracle to 1e-13."""
    import mpmath
    mpmath.mp.dps = digits
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    out = _dec(dec, inp, k, v)
    q = widen_ref(inp["q"], w.dtype)
    G = w.num_q_heads // w.num_kv_heads
    scale = mpmath.mpf(float(np.float32(inp["scale"])))
    worst = 0.0
    for b in range(w.num_seqs):
        L = int(inp["context_lens"][b])
        K = widen_ref(dense_from_chunks(k, inp["block_tables"][b], L), w.dtype)
        V = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
        for h in range(w.num_q_heads):
            g = h // G
            qh = [mpmath.mpf(float(x)) for x in q[b, h]]
            scores = []
            for t in range(L):
                s = mpmath.mpf(0)
                for d in range(w.head_dim):
                    s += qh[d] * mpmath.mpf(float(K[t, g, d]))
                scores.append(s * scale)
            mx = max(scores)
            wts = [mpmath.exp(s - mx) for s in scores]
            tot = mpmath.fsum(wts)
            for d in range(w.head_dim):
                num = mpmath.fsum(wts[t] * mpmath.mpf(float(V[t, g, d]))
                                  for t in range(L))
                worst = max(worst, abs(float(num / tot) - out[b, h, d]))
    return worst <= 1e-13, f"max diff {worst}"


def pin_zero_scale(dec, rac, w):
    """P12: scale 0 makes every weight equal, so out = mean of the V rows."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    out = _dec(dec, inp, k, v, scale=np.float32(0.0))
    G = w.num_q_heads // w.num_kv_heads
    worst = 0.0
    for b in range(w.num_seqs):
        L = int(inp["context_lens"][b])
        V = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
        mean = V.sum(axis=0) / L  # [Hkv, D]
        for h in range(w.num_q_heads):
            worst = max(worst, float(np.max(np.abs(out[b, h] - mean[h // G]))))
    return worst <= 1e-12, f"max diff {worst}"


def pin_poison(dec, rac, w):
    """P13: NaN in every slot no sequence may read (spare blocks, tails of
    last blocks, padded table entries) leaves the output bit-identical."""
    clean = synth.make_inputs(w)
    dirty = synth.make_inputs(w, poison=True)
    kc, vc = written(clean, rac)
    kd, vd = written(dirty, rac)
    a = _dec(dec, clean, kc, vc)
    b = _dec(dec, dirty, kd, vd, block_tables=dirty["block_tables"])
    if not np.array_equal(a, b):
        return False, "poisoned run differs"
    return True, ""


def pin_empty_sequence(dec, rac, w):
    """Reading taken: a sequence of length 0 yields a zero row; the others are
    unaffected by it."""
    ctx = synth.make_inputs(w)["context_lens"].copy()
    ctx[0] = 0
    inp = synth.make_inputs(w, context_lens=ctx)
    k, v = written(inp, rac)
    out = _dec(dec, inp, k, v)
    if np.any(out[0] != 0):
        return False, "row of empty sequence not zero"
    # the other rows are checked against SDPA
    q = widen_ref(inp["q"], w.dtype)
    for b in range(1, w.num_seqs):
        L = int(ctx[b])
        K = widen_ref(dense_from_chunks(k, inp["block_tables"][b], L), w.dtype)
        V = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
        ref = sdpa_ref(q[b], K, V, np.float64(inp["scale"]))
        if np.max(np.abs(out[b] - ref)) > 1e-12:
            return False, f"seq {b} wrong"
    return True, ""


# ---------------------------------------------------------------- shared blocks
def pin_copy_blocks(copy, inp, pairs):
    """P15: after the copy, the rows of each destination block equal the rows
    its source block held, bit for bit; blocks that are no destination keep
    their bits; pairs naming a block outside the pool change nothing.

    Expected values come from the flat-slot view ([num_blocks * bs, ...]):
    block n is flat rows n*bs .. n*bs+bs-1 (row-major layout).  ``pairs``
    must not chain (no block is both a source and a destination).
    """
    kc, vc = inp["k_cache"], inp["v_cache"]
    nb, bs = kc.shape[:2]
    k2, v2 = copy(kc, vc, pairs)
    for old, new in ((kc, k2), (vc, v2)):
        flat_old = old.reshape((nb * bs,) + old.shape[2:])
        flat_new = new.reshape((nb * bs,) + new.shape[2:])
        dest = np.zeros(nb * bs, dtype=bool)
        for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
            if not (0 <= src < nb and 0 <= dst < nb):
                continue
            rows = slice(dst * bs, dst * bs + bs)
            dest[rows] = True
            if flat_new[rows].tobytes() != flat_old[src * bs:src * bs + bs].tobytes():
                return False, f"block {dst} is not a copy of block {src}"
        if flat_new[~dest].tobytes() != flat_old[~dest].tobytes():
            return False, "a block that is no destination changed"
    return True, ""


def pin_shared_prefix(dec, rac, w, members=(0, 1, 2), prefix_blocks=2):
    """P16: sequences whose tables name the same physical blocks for a common
    prefix decode exactly as if each held its own copy of those blocks
    (paging only changes where rows live).  The private copies are made by
    gathering the shared rows chunk by chunk and storing them in fresh
    blocks, independently of the oracle's block copy."""
    inp = synth.make_inputs(w)
    k, v = written(inp, rac)
    tables = inp["block_tables"].copy()
    ctx = inp["context_lens"]
    bs = w.block_size
    lead = members[0]
    for b in members:
        if int(ctx[b]) <= prefix_blocks * bs:
            return False, f"member {b} too short for the shared prefix"
    shared = tables.copy()
    for b in members[1:]:
        shared[b, :prefix_blocks] = tables[lead, :prefix_blocks]
    out_shared = _dec(dec, inp, k, v, block_tables=shared)
    # Private copies: append one fresh block per (member, prefix block).
    extra = len(members[1:]) * prefix_blocks
    k2 = np.concatenate([k, np.zeros((extra,) + k.shape[1:], k.dtype)])
    v2 = np.concatenate([v, np.zeros((extra,) + v.shape[1:], v.dtype)])
    private = shared.copy()
    nxt = k.shape[0]
    for b in members[1:]:
        rows_k = dense_from_chunks(k, tables[lead], prefix_blocks * bs)
        rows_v = dense_from_chunks(v, tables[lead], prefix_blocks * bs)
        for j in range(prefix_blocks):
            k2[nxt] = rows_k[j * bs:(j + 1) * bs]
            v2[nxt] = rows_v[j * bs:(j + 1) * bs]
            private[b, j] = nxt
            nxt += 1
    out_private = _dec(dec, inp, k2, v2, block_tables=private)
    if not np.array_equal(out_shared, out_private):
        return False, "aliased prefix blocks change the result"
    return True, ""


# ---------------------------------------------------------------- prefill
def _prefill(pf, inp, **over):
    args = dict(q=inp["q"], k_cache=inp["k_cache"], v_cache=inp["v_cache"],
                block_tables=inp["block_tables"], context_lens=inp["context_lens"],
                query_start=inp["query_start"], scale=inp["scale"],
                dtype=inp["workload"].dtype)
    args.update(over)
    return pf(args["q"], args["k_cache"], args["v_cache"], args["block_tables"],
              args["context_lens"], args["query_start"], args["scale"], args["dtype"])


def written_prefill(inp, rac):
    return rac(inp["key"], inp["value"], inp["k_cache"], inp["v_cache"],
               inp["slot_mapping"])


def pin_prefill_is_decode_per_token(pf, dec, rac, inp):
    """P17: each new row equals a one-sequence decode whose context ends at
    that row's position (prefill is decode repeated as the context grows)."""
    k, v = written_prefill(inp, rac)
    out = _prefill(pf, inp, k_cache=k, v_cache=v)
    ctx, start = inp["context_lens"], inp["query_start"]
    w = inp["workload"]
    for b in range(len(ctx)):
        n = int(start[b + 1] - start[b])
        for i in range(n):
            row = int(start[b]) + i
            pos = int(ctx[b]) - n + i
            ref = dec(inp["q"][row:row + 1], k, v, inp["block_tables"][b:b + 1],
                      np.array([pos + 1], dtype=np.int32), inp["scale"], w.dtype)
            if not np.array_equal(out[row], ref[0]):
                return False, f"seq {b} row {i}"
    return True, ""


def pin_prefill_causal_sdpa(pf, rac, inp):
    """P18: a whole-prompt prefill equals torch SDPA with is_causal=True
    (CPU, float64) over the sequence's rows gathered chunk by chunk."""
    import torch
    k, v = written_prefill(inp, rac)
    out = _prefill(pf, inp, k_cache=k, v_cache=v)
    w = inp["workload"]
    ctx, start = inp["context_lens"], inp["query_start"]
    for b in range(len(ctx)):
        L = int(ctx[b])
        if int(start[b + 1] - start[b]) != L:
            return False, "not a whole-prompt batch"
        K = widen_ref(dense_from_chunks(k, inp["block_tables"][b], L), w.dtype)
        V = widen_ref(dense_from_chunks(v, inp["block_tables"][b], L), w.dtype)
        Q = widen_ref(inp["q"][int(start[b]):int(start[b + 1])], w.dtype)  # [L, Hq, D]
        rep = w.num_q_heads // w.num_kv_heads
        qt = torch.from_numpy(Q).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(rep, dim=0).unsqueeze(0)
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(rep, dim=0).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt.contiguous(), kt.contiguous(), vt.contiguous(), is_causal=True,
            scale=float(np.float32(inp["scale"]))).squeeze(0).permute(1, 0, 2).numpy()
        if not np.allclose(out[int(start[b]):int(start[b + 1])], ref, rtol=1e-12, atol=1e-12):
            return False, f"seq {b}: max diff {np.abs(out[int(start[b]):int(start[b+1])] - ref).max()}"
    return True, ""


def pin_prefill_chunk_equals_tail(pf, rac, inp, tail):
    """P19: prefilling only the last ``tail[b]`` tokens of each prompt (a chunk
    after a cached prefix) gives exactly the last ``tail[b]`` rows of the
    whole-prompt prefill.  ``inp`` is a whole-prompt batch."""
    k, v = written_prefill(inp, rac)
    full = _prefill(pf, inp, k_cache=k, v_cache=v)
    start = inp["query_start"]
    rows, st = [], [0]
    for b in range(len(start) - 1):
        hi = int(start[b + 1])
        n = min(int(tail[b]), hi - int(start[b]))
        rows.extend(range(hi - n, hi))
        st.append(st[-1] + n)
    rows = np.array(rows, dtype=np.int64)
    out = _prefill(pf, inp, q=inp["q"][rows], k_cache=k, v_cache=v,
                   query_start=np.array(st, dtype=np.int32))
    if not np.array_equal(out, full[rows]):
        return False, "chunk rows differ from the whole prompt's"
    return True, ""


def pin_prefill_first_token(pf, rac, w):
    """P20: a one-token prompt attends to itself only: its output is exactly
    its own V row (softmax of one score is 1)."""
    ctx = np.ones(w.num_seqs, dtype=np.int32)
    inp = synth.make_prefill_inputs(w, context_lens=ctx, query_lens=ctx)
    k, v = written_prefill(inp, rac)
    out = _prefill(pf, inp, k_cache=k, v_cache=v)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        vrow = widen_ref(inp["value"][b], w.dtype)
        for h in range(w.num_q_heads):
            if not np.array_equal(out[b, h], vrow[h // G]):
                return False, f"b={b} h={h}"
    return True, ""
