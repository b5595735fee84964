"""Pins for the fp64 oracle: checks against things other than itself.

Every check takes the oracle module as an argument so that the mutation suite
can run the same checks against deliberately broken copies of the oracle and
confirm that each planted mistake is caught.

What pins what:
  * brute force -- pure-Python textbook attention on contiguous rows (no
    paging, no numpy) on tiny inputs, agreement to 1e-12: pins the gather, the
    GQA head mapping, the scale, the softmax and the causal alignment;
  * closed forms -- one visible key returns its value row exactly; a zero
    query averages the visible values; two worked examples under
    tests/golden (hand-derived from the definition of softmax attention);
  * a library special case -- torch's scaled_dot_product_attention in float64
    on contiguous rows with an explicit bottom-right mask and head repetition;
  * the pages' invariants -- identical output across block sizes 1/4/16/256
    ("mini-vLLM", walls list: parity across KV block sizes), under a
    permutation of physical block IDs ("nano-vLLM Part 4", section 2: tables
    hold physical IDs), and for a sequence batched versus alone ("mini-vLLM",
    project summary: batched output is tested against running alone);
  * cross-path identities -- prefill row i equals a decode over Lk - Lq + i + 1
    keys; a prefill with a cached prefix equals the last rows of a prefill
    that recomputes the prefix;
  * the store -- byte-exact round trip, untouched bytes unchanged, negative
    slots skipped.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import brute_force as BF
from synth import (DecodeSpec, PrefillSpec, decode_subset, logical_prefix, make_decode,
                   make_prefill, prefill_subset)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TINY_DEC_F32 = DecodeSpec("pin-decode-f32", 4, 2, 8, "f32", 4, context_lens=(1, 3, 7, 12))
TINY_DEC_BF16 = DecodeSpec("pin-decode-bf16", 6, 2, 8, "bf16", 4, context_lens=(2, 9, 16))
TINY_PRE_F32 = PrefillSpec("pin-prefill-f32", 4, 2, 8, "f32", 4, q_len_range=(1, 1),
                           q_lens=(1, 5, 9, 0), prefix_lens=(0, 3, 6, 2))
TINY_PRE_BF16 = PrefillSpec("pin-prefill-bf16", 6, 3, 8, "bf16", 4, q_len_range=(1, 1),
                            q_lens=(4, 7), prefix_lens=(5, 0))
SHARED_PRE = PrefillSpec("pin-prefill-shared", 4, 1, 8, "bf16", 4, q_len_range=(1, 6),
                         num_seqs=3, prefix_len=8, shared_prefix=True)


def _store(O, c):
    return O.store_kv(c.k_cache, c.v_cache, c.k_new, c.v_new, c.slot_mapping)


def _decode(O, c):
    kc, vc = _store(O, c)
    return O.decode(c.q, kc, vc, c.block_tables, c.context_lens, c.scale, c.dtype)


def _prefill(O, c):
    kc, vc = _store(O, c)
    return O.prefill_varlen(c.q, kc, vc, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k,
                            c.scale, c.dtype)


def _decode_logical(c, b):
    """Contiguous K/V rows of decode sequence b: history then the new token."""
    lo, hi = c.hist_off[b], c.hist_off[b + 1]
    k = np.concatenate([c.hist_k[lo:hi], c.k_new[b:b + 1]])
    v = np.concatenate([c.hist_v[lo:hi], c.v_new[b:b + 1]])
    return k, v


def _prefill_logical(c, b):
    pk, pv = logical_prefix(c, b)
    q0, q1 = c.cu_seqlens_q[b], c.cu_seqlens_q[b + 1]
    return np.concatenate([pk, c.k_new[q0:q1]]), np.concatenate([pv, c.v_new[q0:q1]])


def _nested(a, dtype):
    if a.ndim == 1:
        return BF.row(a, dtype)
    return [_nested(x, dtype) for x in a]


# ----------------------------------------------------------------------------- brute force

def check_decode_brute_force(O):
    for spec, seed in ((TINY_DEC_F32, 11), (TINY_DEC_BF16, 12)):
        c = make_decode(spec, seed)
        out = _decode(O, c)
        scale = float(c.scale)
        for b in range(c.num_seqs):
            k, v = _decode_logical(c, b)
            exp = BF.decode_seq(_nested(c.q[b], c.dtype), _nested(k, c.dtype),
                                _nested(v, c.dtype), c.num_kv_heads, scale)
            err = np.abs(out[b] - np.asarray(exp)).max()
            assert err < 1e-12, f"{spec.name} seq {b}: {err}"


def check_prefill_brute_force(O):
    for spec, seed in ((TINY_PRE_F32, 21), (TINY_PRE_BF16, 22), (SHARED_PRE, 23)):
        c = make_prefill(spec, seed)
        out = _prefill(O, c)
        scale = float(c.scale)
        for b in range(c.num_seqs):
            q0, q1 = c.cu_seqlens_q[b], c.cu_seqlens_q[b + 1]
            if q1 == q0:
                continue
            k, v = _prefill_logical(c, b)
            exp = BF.prefill_seq(_nested(c.q[q0:q1], c.dtype), _nested(k, c.dtype),
                                 _nested(v, c.dtype), c.num_kv_heads, scale)
            err = np.abs(out[q0:q1] - np.asarray(exp)).max()
            assert err < 1e-12, f"{spec.name} seq {b}: {err}"


# ----------------------------------------------------------------------------- closed forms

def check_single_key_returns_value(O):
    """One visible key: its softmax weight is exactly 1, so the output is that
    key's value row, bit for bit (decode with L = 1; prefill row 0 without prefix)."""
    spec = DecodeSpec("pin-one", 4, 2, 8, "bf16", 4, context_lens=(1, 1, 1))
    c = make_decode(spec, 31)
    out = _decode(O, c)
    g = np.arange(4) // 2
    for b in range(3):
        val = BF.row(c.v_new[b].reshape(-1), c.dtype)
        expect = np.asarray(val).reshape(2, 8)[g]
        assert np.array_equal(out[b], expect), "L=1 decode must return V"
    pc = make_prefill(TINY_PRE_F32, 32)
    pout = _prefill(O, pc)
    b = int(np.flatnonzero((pc.prefix_lens == 0) & (pc.q_lens > 0))[0])
    r0 = pc.cu_seqlens_q[b]
    expect = np.asarray(BF.row(pc.v_new[r0].reshape(-1), pc.dtype)).reshape(
        pc.num_kv_heads, -1)[np.arange(pc.num_q_heads) // (pc.num_q_heads // pc.num_kv_heads)]
    assert np.array_equal(pout[r0], expect), "prefill row 0 without prefix must return V[0]"


def check_zero_query_averages(O):
    """q = 0 makes every score 0, so every visible key weighs the same."""
    c = make_decode(TINY_DEC_F32, 33)
    c.q[:] = 0
    out = _decode(O, c)
    group = c.num_q_heads // c.num_kv_heads
    for b in range(c.num_seqs):
        _, v = _decode_logical(c, b)
        mean = np.asarray(_nested(v, c.dtype)).mean(axis=0)        # [Hkv, D]
        for h in range(c.num_q_heads):
            assert np.abs(out[b, h] - mean[h // group]).max() < 1e-12


def _manual_pool(keys, values, block_size, perm):
    """Lay contiguous rows [L, 1, D] into a pool with the given block order."""
    L, D = len(keys), len(keys[0])
    nblk = -(-L // block_size)
    pool_k = np.full((len(perm), block_size, 1, D), np.nan, np.float32)
    pool_v = np.full_like(pool_k, np.nan)
    table = np.asarray(perm[:nblk], np.int32)
    for j in range(L):
        pool_k[table[j // block_size], j % block_size, 0] = keys[j]
        pool_v[table[j // block_size], j % block_size, 0] = values[j]
    return pool_k, pool_v, table


def check_golden_worked_examples(O):
    """Hand-worked examples (tests/golden): the stored decimals must equal the
    closed form, and the oracle must reproduce them."""
    with open(os.path.join(GOLDEN, "two_key_decode.json")) as f:
        g = json.load(f)
    e2 = math.exp(2.0)
    assert abs(g["expected"][0] - e2 / (1 + e2)) < 1e-15
    assert abs(g["expected"][1] - 1 / (1 + e2)) < 1e-15
    pk, pv, table = _manual_pool(g["keys"], g["values"], 1, [3, 0, 2, 1])
    q = np.asarray([[g["query"]]], np.float32)                       # [1, 1, D]
    out = O.decode(q, pk, pv, table[None, :], np.asarray([len(g["keys"])], np.int32),
                   np.float32(g["scale"]), "f32")
    assert np.abs(out[0, 0] - np.asarray(g["expected"])).max() < 1e-14

    with open(os.path.join(GOLDEN, "three_token_causal_prefill.json")) as f:
        g = json.load(f)
    e = math.e
    closed = [1.0, (1 + 2 * e) / (1 + e), (1 + 2 * e + 3 * e * e) / (1 + e + e * e)]
    assert np.abs(np.asarray(g["expected_rows"]) - closed).max() < 1e-15
    pk, pv, table = _manual_pool(g["keys"], g["values"], 2, [1, 0])
    for case in g["cases"]:
        lq, lk = case["num_new"], len(g["keys"])
        q = np.asarray(g["queries"][lk - lq:], np.float32)[:, None, :]   # [Lq, 1, D]
        out = O.prefill_varlen(q, pk, pv, table[None, :], np.asarray([0, lq], np.int32),
                               np.asarray([0, lk], np.int32), np.float32(g["scale"]), "f32")
        want = np.asarray(case["expected"])
        assert np.abs(out[:, 0, 0] - want).max() < 1e-14, case


def check_gqa_head_mapping(O):
    """Contiguous query groups: with KV head g's values all equal to g + 1,
    query head h must return h // (Hq / Hkv) + 1 everywhere."""
    spec = DecodeSpec("pin-gqa", 6, 3, 8, "f32", 4, context_lens=(3, 6))
    c = make_decode(spec, 34)
    for g in range(3):
        c.v_cache[:, :, g, :] = g + 1.0
        c.v_new[:, g, :] = g + 1.0
    out = _decode(O, c)
    for h in range(6):
        assert np.allclose(out[:, h, :], h // 2 + 1.0, rtol=0, atol=1e-12), h


# ----------------------------------------------------------------------------- library case

def check_torch_sdpa(O):
    """torch's scaled_dot_product_attention in float64 on the contiguous rows,
    KV heads repeated per query group, explicit bottom-right causal mask."""
    import torch
    import torch.nn.functional as F

    def widen(a, dtype):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bf16":
            return t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
        return t.to(torch.float64)

    dspec = DecodeSpec("pin-sdpa-dec", 8, 2, 16, "bf16", 8, num_seqs=3, len_range=(1, 40))
    c = make_decode(dspec, 35)
    out = _decode(O, c)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.num_seqs):
        k, v = _decode_logical(c, b)
        K = widen(k, c.dtype).permute(1, 0, 2).repeat_interleave(G, 0)[None]   # [1,Hq,L,D]
        V = widen(v, c.dtype).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        Q = widen(c.q[b], c.dtype)[None, :, None, :]                             # [1,Hq,1,D]
        ref = F.scaled_dot_product_attention(Q, K, V, scale=float(c.scale))[0, :, 0]
        assert np.abs(out[b] - ref.numpy()).max() < 1e-12

    pspec = PrefillSpec("pin-sdpa-pre", 8, 4, 16, "f32", 8, q_len_range=(1, 30), num_seqs=3,
                        prefix_lens=(0, 13, 40))
    c = make_prefill(pspec, 36)
    out = _prefill(O, c)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.num_seqs):
        q0, q1 = c.cu_seqlens_q[b], c.cu_seqlens_q[b + 1]
        k, v = _prefill_logical(c, b)
        lq, lk = q1 - q0, k.shape[0]
        K = widen(k, c.dtype).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        V = widen(v, c.dtype).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        Q = widen(c.q[q0:q1], c.dtype).permute(1, 0, 2)[None]                   # [1,Hq,Lq,D]
        mask = torch.arange(lk)[None, :] <= (lk - lq) + torch.arange(lq)[:, None]
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=float(c.scale))
        assert np.abs(out[q0:q1] - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


# ----------------------------------------------------------------------------- invariants

def check_block_size_invariance(O):
    """Same logical content paged at block sizes 1, 4, 16, 256: identical output."""
    spec = DecodeSpec("pin-bs", 4, 2, 8, "bf16", 16, context_lens=(1, 4, 17, 40, 300))
    outs = [_decode(O, make_decode(spec, 41, block_size=bs)) for bs in (1, 4, 16, 256)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    pspec = PrefillSpec("pin-bs-pre", 4, 2, 8, "f32", 16, q_len_range=(1, 1),
                        q_lens=(3, 20, 1), prefix_lens=(0, 16, 33))
    outs = [_prefill(O, make_prefill(pspec, 42, block_size=bs)) for bs in (1, 4, 16, 256)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def check_permutation_invariance(O):
    """Different physical block IDs for the same content: identical output."""
    spec = DecodeSpec("pin-perm", 4, 2, 8, "f32", 4, context_lens=(5, 9, 13))
    a = _decode(O, make_decode(spec, 43, perm_seed=1))
    b = _decode(O, make_decode(spec, 43, perm_seed=2))
    assert np.array_equal(a, b)
    a = _prefill(O, make_prefill(TINY_PRE_BF16, 44, perm_seed=1))
    b = _prefill(O, make_prefill(TINY_PRE_BF16, 44, perm_seed=2))
    assert np.array_equal(a, b)


def check_batched_vs_alone(O):
    c = make_decode(TINY_DEC_BF16, 45)
    batched = _decode(O, c)
    for b in range(c.num_seqs):
        alone = _decode(O, decode_subset(c, [b], perm_seed=7))
        assert np.array_equal(alone[0], batched[b])
    rev = _decode(O, decode_subset(c, list(range(c.num_seqs))[::-1], perm_seed=8))
    assert np.array_equal(rev[::-1], batched)
    p = make_prefill(TINY_PRE_F32, 46)
    batched = _prefill(O, p)
    for b in range(p.num_seqs):
        alone = _prefill(O, prefill_subset(p, [b], perm_seed=9))
        q0, q1 = p.cu_seqlens_q[b], p.cu_seqlens_q[b + 1]
        assert np.array_equal(alone, batched[q0:q1])


# ----------------------------------------------------------------------------- cross-path

def check_prefill_row_equals_decode(O):
    """Row i of a sequence's new tokens is a decode over its first
    Lk - Lq + i + 1 keys."""
    c = make_prefill(TINY_PRE_BF16, 47)
    kc, vc = _store(O, c)
    out = O.prefill_varlen(c.q, kc, vc, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k,
                           c.scale, c.dtype)
    for b in range(c.num_seqs):
        q0, q1 = c.cu_seqlens_q[b], c.cu_seqlens_q[b + 1]
        lq = q1 - q0
        lk = c.cu_seqlens_k[b + 1] - c.cu_seqlens_k[b]
        for i in range(lq):
            d = O.decode(c.q[q0 + i][None], kc, vc, c.block_tables[b:b + 1],
                         np.asarray([lk - lq + i + 1], np.int32), c.scale, c.dtype)
            assert np.abs(d[0] - out[q0 + i]).max() < 1e-12, (b, i)


def check_prefix_equals_full_suffix(O):
    """With a cached prefix of P tokens, the Lq new rows equal the last Lq
    rows of a prefill that treats all P + Lq tokens as new queries."""
    c = make_prefill(TINY_PRE_F32, 48)
    kc, vc = _store(O, c)
    out = O.prefill_varlen(c.q, kc, vc, c.block_tables, c.cu_seqlens_q, c.cu_seqlens_k,
                           c.scale, c.dtype)
    rng = np.random.default_rng(5)
    klens = np.diff(c.cu_seqlens_k)
    q_full = []
    for b in range(c.num_seqs):
        filler = rng.standard_normal((int(c.prefix_lens[b]), c.num_q_heads, c.head_dim))
        q_full += [filler.astype(np.float32), c.q[c.cu_seqlens_q[b]:c.cu_seqlens_q[b + 1]]]
    q_full = np.concatenate(q_full)
    full = O.prefill_varlen(q_full, kc, vc, c.block_tables, c.cu_seqlens_k, c.cu_seqlens_k,
                            c.scale, c.dtype)
    for b in range(c.num_seqs):
        q0, q1 = c.cu_seqlens_q[b], c.cu_seqlens_q[b + 1]
        k1 = c.cu_seqlens_k[b + 1]
        if q1 == q0:
            continue
        assert np.abs(full[k1 - (q1 - q0):k1] - out[q0:q1]).max() < 1e-12, b
    assert np.all(klens >= np.diff(c.cu_seqlens_q))


# ----------------------------------------------------------------------------- store

def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def check_store_round_trip(O):
    """After the store every written row reads back bit for bit at its slot,
    rows with a negative slot are not written, and no other byte changes."""
    spec = DecodeSpec("pin-store", 4, 2, 8, "bf16", 4, context_lens=(1, 4, 5, 8, 9, 2))
    c = make_decode(spec, 51)
    slots = c.slot_mapping.copy()
    slots[2] = -1                                   # a padding row
    nb, bs = c.num_blocks, c.block_size
    free = np.setdiff1d(np.arange(nb * bs), c.slot_mapping)
    slots[4] = 0 if 0 in free else slots[4]         # exercise slot 0 when it is free
    kc, vc = O.store_kv(c.k_cache, c.v_cache, c.k_new, c.v_new, slots)
    for pool_before, pool_after, rows in ((c.k_cache, kc, c.k_new), (c.v_cache, vc, c.v_new)):
        before = _bits(pool_before).reshape(nb * bs, -1)
        after = _bits(pool_after).reshape(nb * bs, -1)
        src = _bits(rows).reshape(len(slots), -1)
        written = slots[slots >= 0]
        for t, s in enumerate(slots):
            if s >= 0:
                assert np.array_equal(after[s], src[t]), (t, s)
        keep = np.setdiff1d(np.arange(nb * bs), written)
        assert np.array_equal(after[keep], before[keep])
    # the skipped row's content appears nowhere it was not already
    skipped = _bits(c.k_new[2]).reshape(-1)
    after = _bits(kc).reshape(nb * bs, -1)
    before = _bits(c.k_cache).reshape(nb * bs, -1)
    hits_after = np.all(after == skipped, axis=1).sum()
    hits_before = np.all(before == skipped, axis=1).sum()
    assert hits_after == hits_before


def check_store_f32_and_zero_slot(O):
    spec = DecodeSpec("pin-store-f32", 2, 1, 4, "f32", 2, context_lens=(1, 2, 3))
    c = make_decode(spec, 52)
    slots = np.asarray([0, 3, 5], np.int32)        # fixed slots, slot 0 included
    kc, vc = O.store_kv(c.k_cache, c.v_cache, c.k_new, c.v_new, slots)
    for t, s in enumerate(slots):
        assert np.array_equal(_bits(kc[s // 2, s % 2]), _bits(c.k_new[t]))
        assert np.array_equal(_bits(vc[s // 2, s % 2]), _bits(c.v_new[t]))


ALL_CHECKS = [
    check_decode_brute_force, check_prefill_brute_force, check_single_key_returns_value,
    check_zero_query_averages, check_golden_worked_examples, check_gqa_head_mapping,
    check_torch_sdpa, check_block_size_invariance, check_permutation_invariance,
    check_batched_vs_alone, check_prefill_row_equals_decode, check_prefix_equals_full_suffix,
    check_store_round_trip, check_store_f32_and_zero_slot,
]
