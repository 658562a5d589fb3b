"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of one oracle function with one plausible bug (a dropped
term, a wrong sign or index, a transposed operand).  The test runs the pins
that exercise that function and requires at least one to fail, which shows the
pins constrain every part of the oracle rather than only agreeing with it.
"""
import numpy as np
import pytest

import oracle
from oracle import paged_attention as PA
import synth
from tests import _pins as P

W_F32 = synth.WORKLOADS["tiny_f32"]
W_BF16 = synth.Workload("gqa4_bf16", 6, 8, 2, 32, 16, "bf16",
                        ("uniform", 1, 100), num_blocks=48, seed=21)


def _decode_one_factory(kind):
    def decode_one(q_b, K, V, scale):
        Hq, D = q_b.shape
        L, Hkv, _ = K.shape
        if L == 0:
            return np.zeros((Hq, D))
        group = Hq // Hkv
        kv_head = np.arange(Hq) // group
        if kind == "gqa_modulo":
            kv_head = np.arange(Hq) % Hkv
        Kh = K[:, kv_head, :]
        Vh = V[:, kv_head, :]
        if kind == "k_v_swapped":
            Kh, Vh = Vh, Kh
        sc = np.float64(scale)
        if kind == "no_scale":
            sc = 1.0
        if kind == "scale_squared":
            sc = sc * sc
        s = sc * np.einsum("hd,thd->ht", q_b, Kh)
        if kind == "sign":
            s = -s
        m = s.max(axis=1, keepdims=True)
        if kind == "no_max":
            m = 0.0
        p = np.exp(s - m)
        if kind == "drop_last":
            p[:, -1] = 0.0 if L > 1 else p[:, -1]
        num = np.einsum("ht,thd->hd", p, Vh)
        if kind == "no_norm":
            return num
        if kind == "norm_by_count":
            return num / L
        return num / p.sum(axis=1)[:, None]
    return decode_one


def _decode_factory(kind):
    """Mutants of the paged lookup inside decode."""
    def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
        scale = np.float64(np.float32(scale))
        qf = PA.widen(q, dtype)
        bs = k_cache.shape[1]
        out = np.zeros(qf.shape)
        for b in range(qf.shape[0]):
            L = int(context_lens[b])
            if kind == "ctx_minus_one":
                L -= 1
            if kind == "whole_blocks":
                L = -(-L // bs) * bs
            if L <= 0:
                continue
            pos = np.arange(L)
            blk = pos // bs
            off = pos % bs
            if kind == "offset_reversed":
                off = bs - 1 - off
            if kind == "table_transposed":
                # column-major index into the row-major table
                phys = block_tables.reshape(-1)[(blk * block_tables.shape[0] + b)
                                                % block_tables.size]
            else:
                phys = block_tables[b, blk]
            phys = phys.astype(np.int64)
            K = PA.widen(k_cache[phys, off], dtype)
            V = PA.widen(v_cache[phys, off], dtype)
            out[b] = PA.decode_one(qf[b], K, V, scale)
        return out
    return decode


def _rac_factory(kind):
    def rac(key, value, k_cache, v_cache, slot_mapping):
        k_out = np.array(k_cache, copy=True)
        v_out = np.array(v_cache, copy=True)
        bs = k_cache.shape[1]
        for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
            slot = int(slot)
            if slot < 0 and kind != "no_skip":
                continue
            blk, off = slot // bs, slot % bs
            if kind == "off_by_one":
                off = (off + 1) % bs
            k_out[blk, off] = key[i]
            if kind == "v_gets_k":
                v_out[blk, off] = key[i]
            elif kind != "k_only":
                v_out[blk, off] = value[i]
        return k_out, v_out
    return rac


def _merge_factory(kind):
    def merge(m, l, acc):
        B, Hq, Pn = m.shape
        out = np.zeros(acc.shape[:2] + acc.shape[3:])
        for b in range(B):
            for h in range(Hq):
                valid = np.isfinite(m[b, h])
                if not valid.any():
                    continue
                M = m[b, h, valid].max()
                w = np.exp(m[b, h, valid] - M)
                Lsum = (l[b, h, valid] * (1.0 if kind == "l_unweighted" else w)).sum()
                if kind == "acc_unweighted":
                    w = np.ones_like(w)
                out[b, h] = (acc[b, h, valid] * w[:, None]).sum(axis=0) / Lsum
        return out
    return merge


def _decode_pins(dec, rac=oracle.reshape_and_cache):
    yield P.pin_single_token(dec, rac, W_F32)
    yield P.pin_single_token(dec, rac, W_BF16)
    yield P.pin_block_permutation(dec, rac, W_BF16)
    yield P.pin_gqa_equals_mha(dec, rac, W_BF16)
    yield P.pin_contiguous(dec, rac, W_BF16)
    yield P.pin_zero_scale(dec, rac, W_BF16)
    yield P.pin_onehot(dec, W_F32)
    yield P.pin_uncached_recompute(dec, rac)
    yield P.pin_sdpa(dec, rac, W_F32)
    yield P.pin_sdpa(dec, rac, W_BF16)


def _first_failure(results):
    for ok, detail in results:
        if not ok:
            return detail
    return None


@pytest.mark.parametrize("kind", ["gqa_modulo", "k_v_swapped", "no_scale",
                                  "scale_squared", "sign", "no_max", "drop_last",
                                  "no_norm", "norm_by_count"])
def test_decode_math_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(PA, "decode_one", _decode_one_factory(kind))
    with np.errstate(all="ignore"):
        caught = _first_failure(_decode_pins(oracle.decode))
    assert caught is not None, f"mutant {kind} passed every pin"


@pytest.mark.parametrize("kind", ["ctx_minus_one", "whole_blocks",
                                  "offset_reversed", "table_transposed"])
def test_decode_lookup_mutant_is_caught(kind):
    dec = _decode_factory(kind)
    with np.errstate(all="ignore"):
        caught = _first_failure(_decode_pins(dec))
    assert caught is not None, f"mutant {kind} passed every pin"


@pytest.mark.parametrize("kind", ["no_skip", "off_by_one", "v_gets_k", "k_only"])
def test_write_mutant_is_caught(kind):
    inp = synth.make_inputs(W_BF16)
    inp["slot_mapping"][2] = -1
    ok, _ = P.pin_write_slots(_rac_factory(kind), inp)
    assert not ok


@pytest.mark.parametrize("kind", ["l_unweighted", "acc_unweighted"])
def test_merge_mutant_is_caught(kind):
    ok, _ = P.pin_split_merge(oracle.decode, oracle.decode_partials,
                              _merge_factory(kind), oracle.reshape_and_cache,
                              W_BF16, 16)
    assert not ok


def test_gather_mutant_is_caught():
    def gather_no_zero(cache, block_tables, context_lens):
        g = oracle.gather_kv(cache, block_tables, context_lens)
        g[:, -1] = cache[0, 0]
        return g
    ok, _ = P.pin_gather_chunks(gather_no_zero, synth.make_inputs(W_BF16))
    assert not ok


@pytest.mark.parametrize("kind", ["k_only", "swapped", "no_bounds"])
def test_copy_mutant_is_caught(kind):
    def copy(k_cache, v_cache, block_pairs):
        k_out, v_out = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
        nb = k_cache.shape[0]
        for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
            if kind != "no_bounds" and not (0 <= src < nb and 0 <= dst < nb):
                continue
            if kind == "swapped":
                src, dst = dst, src
            k_out[dst % nb] = k_out[src % nb]
            if kind != "k_only":
                v_out[dst % nb] = v_out[src % nb]
        return k_out, v_out
    inp = synth.make_inputs(W_BF16)
    nb = inp["num_blocks"]
    pairs = np.array([[1, nb - 1], [3, 0], [-1, 2], [2, nb]], dtype=np.int64)
    ok, _ = P.pin_copy_blocks(copy, inp, pairs)
    assert not ok



def _prefill_factory(kind):
    def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype):
        scale = np.float64(np.float32(scale))
        qf = PA.widen(q, dtype)
        out = np.zeros(qf.shape)
        bs = k_cache.shape[1]
        for b in range(len(context_lens)):
            L = int(context_lens[b])
            lo, hi = int(query_start[b]), int(query_start[b + 1])
            n = hi - lo
            pos = np.arange(L)
            phys = block_tables[b, pos // bs].astype(np.int64)
            K = PA.widen(k_cache[phys, pos % bs], dtype)
            V = PA.widen(v_cache[phys, pos % bs], dtype)
            for i in range(n):
                p = L - n + i
                end = {"offset_from_zero": i + 1, "excludes_self": p,
                       "one_ahead": min(L, p + 2), "not_causal": L}.get(kind, p + 1)
                out[lo + i] = PA.decode_one(qf[lo + i], K[:end], V[:end], scale)
        return out
    return prefill


PF_W = synth.Workload("pf_gqa2_bf16", 3, 4, 2, 32, 16, "bf16", ("uniform", 20, 70),
                      seed=31, query=("uniform", 2, 40))
PF_FULL = synth.Workload("pf_full_f32", 2, 2, 2, 16, 16, "f32", ("uniform", 10, 40),
                         seed=32, query=("full",))


@pytest.mark.parametrize("kind", ["offset_from_zero", "excludes_self", "one_ahead",
                                  "not_causal"])
def test_prefill_mutant_is_caught(kind):
    pf = _prefill_factory(kind)
    results = [
        P.pin_prefill_is_decode_per_token(pf, oracle.decode, oracle.reshape_and_cache,
                                          synth.make_prefill_inputs(PF_W)),
        P.pin_prefill_causal_sdpa(pf, oracle.reshape_and_cache,
                                  synth.make_prefill_inputs(PF_FULL)),
    ]
    assert not all(ok for ok, _ in results)
