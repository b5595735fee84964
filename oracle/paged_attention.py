"""fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing but the tests, the package smoke check and
the benchmark's CPU-baseline leg may import or call this module.  The GPU path
(the HIP library and its Python binding) never calls it, and the two share no
code: not a kernel, header, helper, constant or table.

What it computes, and where the pages say so:

* store -- each new token's K and V row is copied to the physical slot the
  slot mapping names ("nano-vLLM Part 4", section 3, prefill/decode table: K/V
  is written for every new prompt token, or for one token per sequence in
  decode; the smzdm Nano-vLLM walk-through, section on model implementation
  details: the store kernel writes K and V to their physical position).
* gather -- logical token j of a sequence is read from block
  ``block_table[j // block_size]`` at offset ``j % block_size`` ("nano-vLLM
  Part 4", section 2: the block table holds physical block IDs).
* decode -- one query token per sequence attends to that sequence's whole
  cached history ("mini-vLLM", project summary; "nano-vLLM Part 4", section 3:
  decode attention runs over the cached history through the block table).
* varlen prefill -- prompts laid end to end in one batch; a row sees only
  keys of its own prompt at or before its own position ("mini-vLLM", project
  summary).  When a sequence has more keys than new
  queries (cu_seqlens_k > cu_seqlens_q: a prefix-cache hit, smzdm walk-through,
  model implementation details) the new rows are the LAST rows of the
  sequence, so row i sees keys 0 .. (Lk - Lq) + i (bottom-right alignment).
* grouped-query attention: query head h reads KV head h // (Hq / Hkv)
  (contiguous groups; "mini-vLLM" names grouped-query attention but not the
  mapping -- this is the plain reading).

Attention itself is the textbook definition, evaluated in float64 on the
exact values the GPU receives (bf16 bit patterns or float32, widened without
rounding): scores = scale * <q, k>, softmax over the visible keys (the maximum
is subtracted first, which changes no value in exact arithmetic), output =
softmax-weighted sum of value rows.  Paging changes addresses, never values.

Pins (all in the CPU test suite): pure-Python brute force on contiguous K/V,
closed forms (one key; zero query; equal keys; a two-key example worked by
hand), torch's scaled_dot_product_attention in float64 with an explicit mask,
invariance under block size 1/4/16/256, block-ID permutation and batching,
prefill/decode cross-checks, byte-exact store round trips, and a mutation
suite that plants plausible mistakes here and checks that a pin fails.
"""
from __future__ import annotations

import numpy as np

__all__ = ["widen", "store_kv", "gather", "decode", "prefill_varlen"]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements.  'bf16' arrays carry raw
    bfloat16 bit patterns (uint16): the bits are the upper half of a float32."""
    if dtype == "bf16":
        as_f32 = (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32)
        return as_f32.astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def store_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
             slot_mapping: np.ndarray):
    """Pools after the store: a copy of the inputs in which row t of k / v is
    placed at slot ``slot_mapping[t]``; a negative slot means "no write" (a
    padding row).  Pools are ``[num_blocks, block_size, kv_heads, head_dim]``;
    rows are copied bit for bit."""
    bs = k_cache.shape[1]
    kc = k_cache.copy()
    vc = v_cache.copy()
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        kc[s // bs, s % bs] = k[t]
        vc[s // bs, s % bs] = v[t]
    return kc, vc


def gather(pool: np.ndarray, table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """The first n_tokens logical rows of one sequence, ``[n, kv_heads, head_dim]``."""
    bs = pool.shape[1]
    pos = np.arange(n_tokens)
    return pool[table_row[pos // bs], pos % bs]


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale, dtype: str) -> np.ndarray:
    """Decode attention: ``q`` is ``[B, Hq, D]``; sequence b attends over its
    ``context_lens[b]`` cached tokens.  Returns float64 ``[B, Hq, D]``."""
    B, num_q_heads, D = q.shape
    num_kv_heads = k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    scale = float(np.float32(scale))
    out = np.zeros((B, num_q_heads, D), np.float64)
    for b in range(B):
        L = int(context_lens[b])
        keys = widen(gather(k_cache, block_tables[b], L), dtype)      # [L, Hkv, D]
        values = widen(gather(v_cache, block_tables[b], L), dtype)
        for h in range(num_q_heads):
            g = h // group
            q_vec = widen(q[b, h], dtype)
            scores = scale * (keys[:, g, :] @ q_vec)                    # [L]
            m = scores.max()
            p = np.exp(scores - m)
            out[b, h] = (p @ values[:, g, :]) / p.sum()
    return out


def prefill_varlen(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                   block_tables: np.ndarray, cu_seqlens_q: np.ndarray,
                   cu_seqlens_k: np.ndarray, scale, dtype: str) -> np.ndarray:
    """Varlen causal prefill: ``q`` is ``[Tq, Hq, D]`` packed by cu_seqlens_q;
    sequence b has Lq new queries and Lk >= Lq keys (the cached prefix followed
    by the new tokens), all read from the pools.  Returns float64 ``[Tq, Hq, D]``."""
    Tq, num_q_heads, D = q.shape
    num_kv_heads = k_cache.shape[2]
    group = num_q_heads // num_kv_heads
    scale = float(np.float32(scale))
    out = np.zeros((Tq, num_q_heads, D), np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        lq = q1 - q0
        lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if lq == 0:
            continue
        keys = widen(gather(k_cache, block_tables[b], lk), dtype)      # [Lk, Hkv, D]
        values = widen(gather(v_cache, block_tables[b], lk), dtype)
        rows = np.arange(lq)[:, None]
        cols = np.arange(lk)[None, :]
        visible = cols <= (lk - lq) + rows                              # [Lq, Lk]
        for h in range(num_q_heads):
            g = h // group
            qh = widen(q[q0:q1, h, :], dtype)                           # [Lq, D]
            S = scale * (qh @ keys[:, g, :].T)                          # [Lq, Lk]
            S = np.where(visible, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            out[q0:q1, h] = (P @ values[:, g, :]) / P.sum(axis=1, keepdims=True)
    return out
