"""Seeded synthetic inputs for attention over a paged KV cache.

This module draws everything a paged-attention step consumes: sequence
lengths, the physical block IDs a block manager would hand out, N(0, 1) query,
key and value rows rounded to the storage dtype, and the block pool holding
the already-cached history.  It performs no attention arithmetic and no store:
the new rows of the step are returned separately, with the slots the store
must write them to.  Both the fp64 oracle's tests and the GPU path's
tests/bench draw their inputs here; neither of those imports the other.

Data model (the pages' vocabulary):
  * a K pool and a V pool, each ``[num_blocks, block_size, kv_heads, head_dim]``
    ("nano-vLLM Part 4", section 2: one KV-cache tensor per rank, allocated at
    start-up; "mini-vLLM": a preallocated pool of fixed-size token blocks);
  * ``block_tables[b]`` lists the physical block IDs of sequence ``b`` in
    logical order ("nano-vLLM Part 4", section 2: a block table holds IDs, not
    K/V values);
  * logical token ``j`` of sequence ``b`` lives at block
    ``block_tables[b][j // block_size]``, offset ``j % block_size``, so its slot
    is ``block_tables[b][j // block_size] * block_size + j % block_size``.  The
    pages name the slot mapping but do not print it; this is the plain reading.

Storage dtypes: 'f32' arrays are float32; 'bf16' arrays hold raw bfloat16 bit
patterns as uint16 (numpy has no bfloat16), rounded from float32 draws with
round-to-nearest-even.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "DecodeSpec", "PrefillSpec", "DecodeCase", "PrefillCase", "CONFIGS",
    "make_decode", "make_prefill", "make_case", "bf16_bits", "poison_bits",
    "decode_subset", "prefill_subset", "logical_prefix",
    "storage_np_dtype", "token_rows",
]

# Named random streams; each is its own SeedSequence so that changing the
# paging (block size, block-ID permutation) never changes the logical content.
_S_LENGTHS, _S_PREFIX_K, _S_PREFIX_V, _S_HIST_K, _S_HIST_V = 0, 1, 2, 3, 4
_S_NEW_K, _S_NEW_V, _S_Q, _S_PAGING = 5, 6, 7, 8
_S_PROLOGUE = 9
_S_TOKEN_ROWS = 10

_CHUNK = 1 << 22  # elements per independently seeded chunk of a normal draw


def _threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(stream, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def storage_np_dtype(dtype: str):
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normal draws; NaN payloads are not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = u >> 16
    b &= 1
    b += 0x7FFF
    b += u
    b >>= 16
    return b.astype(np.uint16)


def poison_bits(dtype: str, kind: str, which: str):
    """Fill value for pool slots that hold no valid token.

    kind 'nan': quiet NaN; 'big': +1e4 in the K pool and -1e4 in the V pool;
    'zero': 0.  A kernel that lets any of these reach its output is wrong.
    """
    if kind == "nan":
        return np.uint16(0x7FC0) if dtype == "bf16" else np.uint32(0x7FC00000).view(np.float32)
    if kind == "big":
        val = 1.0e4 if which == "k" else -1.0e4
    elif kind == "zero":
        val = 0.0
    else:
        raise ValueError(f"unknown poison {kind!r}")
    if dtype == "bf16":
        return bf16_bits(np.array([val], np.float32))[0]
    return np.float32(val)


def _normal_rows(seed: int, stream: int, n_rows: int, row_shape: Tuple[int, ...],
                 dtype: str) -> np.ndarray:
    """N(0, 1) float32 draws in fixed-size chunks (one seeded generator per
    chunk, so the values do not depend on the thread count), rounded to dtype."""
    row_elems = int(np.prod(row_shape))
    n = n_rows * row_elems
    out = np.empty(n, storage_np_dtype(dtype))
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(i: int) -> None:
        lo = i * _CHUNK
        m = min(_CHUNK, n - lo)
        x = _rng(seed, stream, i).standard_normal(m, dtype=np.float32)
        out[lo:lo + m] = bf16_bits(x) if dtype == "bf16" else x

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape((n_rows,) + tuple(row_shape))


# --------------------------------------------------------------------------- specs

@dataclass(frozen=True)
class DecodeSpec:
    """One decode step: a new token per sequence is stored, then attends over
    its whole context (history plus itself)."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    context_lens: Optional[Tuple[int, ...]] = None   # fixed lengths, or drawn:
    num_seqs: int = 0
    len_range: Tuple[int, int] = (1, 1)              # inclusive bounds
    num_blocks: Optional[int] = None                 # fixed pool size (at block_size)
    free_frac: float = 0.10                          # spare blocks beyond the need


@dataclass(frozen=True)
class PrefillSpec:
    """One prefill step over packed prompts; optionally each sequence already
    has ``prefix_len`` cached tokens (shared physical blocks when
    ``shared_prefix``), so keys run past the new queries."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    q_len_range: Tuple[int, int]                     # inclusive bounds
    token_budget: Optional[int] = None               # pack prompts up to this many tokens
    num_seqs: int = 0                                # or a fixed number of sequences
    q_lens: Optional[Tuple[int, ...]] = None         # or fixed new-token counts
    prefix_len: int = 0
    prefix_lens: Optional[Tuple[int, ...]] = None    # per-sequence cached lengths (private)
    shared_prefix: bool = False
    free_frac: float = 0.10


# The five workloads: shapes of Qwen2.5-0.5B / Qwen3-0.6B attention layers.
CONFIGS = {
    1: DecodeSpec("tiny-decode-f32", 2, 1, 64, "f32", 16,
                  context_lens=(5, 17, 33, 64), num_blocks=32),
    2: DecodeSpec("qwen2.5-0.5b-decode", 14, 2, 64, "bf16", 16,
                  num_seqs=32, len_range=(128, 2048)),
    3: DecodeSpec("qwen3-0.6b-decode", 16, 8, 128, "bf16", 256,
                  num_seqs=256, len_range=(100, 2048)),
    4: PrefillSpec("qwen3-0.6b-varlen-prefill", 16, 8, 128, "bf16", 256,
                   q_len_range=(100, 1024), token_budget=16384),
    5: PrefillSpec("qwen3-0.6b-prefix-prefill", 16, 8, 128, "bf16", 256,
                   q_len_range=(64, 512), num_seqs=64, prefix_len=1024,
                   shared_prefix=True),
}


# --------------------------------------------------------------------------- cases

@dataclass
class DecodeCase:
    spec: DecodeSpec
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray        # int32 [B]; includes the new token
    block_tables: np.ndarray        # int32 [B, MB]
    slot_mapping: np.ndarray        # int32 [B]; slot of the new token (position L-1)
    k_cache: np.ndarray             # [NB, BS, Hkv, D] before the store
    v_cache: np.ndarray
    k_new: np.ndarray               # [B, Hkv, D]
    v_new: np.ndarray
    q: np.ndarray                   # [B, Hq, D]
    scale: np.float32
    hist_k: np.ndarray              # logical history rows [sum(L-1), Hkv, D]
    hist_v: np.ndarray
    hist_off: np.ndarray            # int64 [B+1]
    poison: str = "nan"

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


@dataclass
class PrefillCase:
    spec: PrefillSpec
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    cu_seqlens_q: np.ndarray        # int32 [B+1]
    cu_seqlens_k: np.ndarray        # int32 [B+1]
    block_tables: np.ndarray        # int32 [B, MB]
    slot_mapping: np.ndarray        # int32 [Tq]; slots of the new tokens
    k_cache: np.ndarray             # before the store: cached prefixes only
    v_cache: np.ndarray
    k_new: np.ndarray               # [Tq, Hkv, D]
    v_new: np.ndarray
    q: np.ndarray                   # [Tq, Hq, D]
    scale: np.float32
    prefix_lens: np.ndarray         # int32 [B]
    prefix_k: np.ndarray            # shared: [P, Hkv, D]; private: concatenated
    prefix_v: np.ndarray
    prefix_off: np.ndarray          # int64 [B+1] into prefix_k (private only)
    shared_prefix: bool = False
    poison: str = "nan"

    @property
    def num_seqs(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def k_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_k)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.k_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


# --------------------------------------------------------------------------- paging

def _allocate(rng: np.random.Generator, shared_blocks: int, private_blocks: Sequence[int],
              num_blocks: Optional[int], free_frac: float, width: int = 0):
    """Hand out physical block IDs as a shuffled free list would: a seeded
    permutation of the pool, taken in sequence order.  Returns the block
    tables (unused entries point at a spare block, so a reader that strays
    past a sequence's blocks sees poison instead of faulting) and the pool size."""
    need = shared_blocks + int(sum(private_blocks))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(need * (1.0 + free_frac))))
    if num_blocks < need:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")
    ids = rng.permutation(num_blocks).astype(np.int32)
    shared = ids[:shared_blocks]
    spare = int(ids[need]) if num_blocks > need else int(ids[0])
    nb_max = max([shared_blocks + p for p in private_blocks] + [1, width])
    tables = np.full((len(private_blocks), nb_max), spare, np.int32)
    pos = shared_blocks
    for b, p in enumerate(private_blocks):
        tables[b, :shared_blocks] = shared
        tables[b, shared_blocks:shared_blocks + p] = ids[pos:pos + p]
        pos += p
    return tables, num_blocks


def _slots(tables: np.ndarray, seq: np.ndarray, pos: np.ndarray, bs: int) -> np.ndarray:
    return (tables[seq, pos // bs].astype(np.int64) * bs + pos % bs)


def _empty_pool(nb: int, bs: int, hkv: int, d: int, dtype: str, poison: str, which: str):
    return np.full((nb, bs, hkv, d), poison_bits(dtype, poison, which),
                   dtype=storage_np_dtype(dtype))


def _place(pool: np.ndarray, slots: np.ndarray, rows: np.ndarray) -> None:
    if slots.size:
        nb, bs, hkv, d = pool.shape
        pool.reshape(nb * bs, hkv, d)[slots] = rows


# --------------------------------------------------------------------------- decode

def _page_decode(spec: DecodeSpec, lens: np.ndarray, hist_k, hist_v, k_new, v_new, q,
                 bs: int, perm_seed: int, poison: str, fixed_nb: Optional[int],
                 width: int = 0) -> DecodeCase:
    hkv, d, dt = spec.num_kv_heads, spec.head_dim, spec.dtype
    B = int(lens.size)
    hist_n = lens - 1
    hist_off = np.zeros(B + 1, np.int64)
    np.cumsum(hist_n, out=hist_off[1:])
    per_seq = [int(math.ceil(int(L) / bs)) for L in lens]
    tables, nb = _allocate(_rng(perm_seed, _S_PAGING), 0, per_seq, fixed_nb, spec.free_frac,
                           width)
    seq = np.repeat(np.arange(B), hist_n)
    pos = np.arange(int(hist_off[-1])) - np.repeat(hist_off[:-1], hist_n)
    hslots = _slots(tables, seq, pos, bs)
    k_cache = _empty_pool(nb, bs, hkv, d, dt, poison, "k")
    v_cache = _empty_pool(nb, bs, hkv, d, dt, poison, "v")
    _place(k_cache, hslots, hist_k)
    _place(v_cache, hslots, hist_v)
    new_slots = _slots(tables, np.arange(B), lens - 1, bs).astype(np.int32)
    return DecodeCase(spec=spec, dtype=dt, num_q_heads=spec.num_q_heads, num_kv_heads=hkv,
                      head_dim=d, block_size=bs, num_blocks=nb,
                      context_lens=lens.astype(np.int32), block_tables=tables,
                      slot_mapping=new_slots, k_cache=k_cache, v_cache=v_cache,
                      k_new=k_new, v_new=v_new, q=q, scale=np.float32(1.0 / math.sqrt(d)),
                      hist_k=hist_k, hist_v=hist_v, hist_off=hist_off, poison=poison)


def make_decode(spec: DecodeSpec, seed: int, block_size: Optional[int] = None,
                perm_seed: Optional[int] = None, poison: str = "nan",
                context_lens: Optional[Sequence[int]] = None,
                num_blocks: Optional[int] = None) -> DecodeCase:
    """Draw a decode step.  Draw order: lengths, history K, history V, new K,
    new V, Q (each its own stream); the block permutation comes from
    ``perm_seed`` (default ``seed``) so that re-paging keeps the content.
    The new token of sequence b sits at position ``context_lens[b] - 1``."""
    bs = spec.block_size if block_size is None else block_size
    perm_seed = seed if perm_seed is None else perm_seed
    hq, hkv, d, dt = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if context_lens is not None:
        lens = np.asarray(context_lens, np.int64)
    elif spec.context_lens is not None:
        lens = np.asarray(spec.context_lens, np.int64)
    else:
        lo, hi = spec.len_range
        lens = _rng(seed, _S_LENGTHS).integers(lo, hi, endpoint=True, size=spec.num_seqs)
    if np.any(lens < 1):
        raise ValueError("every context length must be >= 1 (it includes the new token)")
    B = int(lens.size)
    n_hist = int((lens - 1).sum())
    hist_k = _normal_rows(seed, _S_HIST_K, n_hist, (hkv, d), dt)
    hist_v = _normal_rows(seed, _S_HIST_V, n_hist, (hkv, d), dt)
    k_new = _normal_rows(seed, _S_NEW_K, B, (hkv, d), dt)
    v_new = _normal_rows(seed, _S_NEW_V, B, (hkv, d), dt)
    q = _normal_rows(seed, _S_Q, B, (hq, d), dt)
    fixed_nb = num_blocks if num_blocks is not None else (
        spec.num_blocks if bs == spec.block_size else None)
    return _page_decode(spec, lens, hist_k, hist_v, k_new, v_new, q, bs, perm_seed, poison,
                        fixed_nb)


def decode_subset(case: DecodeCase, seqs: Sequence[int], perm_seed: int = 0,
                  block_size: Optional[int] = None, table_width: int = 0) -> DecodeCase:
    """The same sequences (same content, fresh paging), alone or in another
    batch order: the "batched versus alone" comparison of the mini-vLLM page.
    ``table_width`` pads the block tables (with a spare block) to at least
    that many columns."""
    seqs = list(seqs)
    lens = case.context_lens[seqs].astype(np.int64)
    hk = [case.hist_k[case.hist_off[b]:case.hist_off[b + 1]] for b in seqs]
    hv = [case.hist_v[case.hist_off[b]:case.hist_off[b + 1]] for b in seqs]
    hk = np.concatenate(hk) if hk else case.hist_k[:0]
    hv = np.concatenate(hv) if hv else case.hist_v[:0]
    bs = case.block_size if block_size is None else block_size
    return _page_decode(case.spec, lens, hk, hv, case.k_new[seqs].copy(),
                        case.v_new[seqs].copy(), case.q[seqs].copy(), bs, perm_seed,
                        case.poison, None, table_width)


# --------------------------------------------------------------------------- prefill

def _page_prefill(spec: PrefillSpec, ql: np.ndarray, pl: np.ndarray, shared: bool,
                  prefix_k, prefix_v, prefix_off, k_new, v_new, q, bs: int, perm_seed: int,
                  poison: str, width: int = 0) -> PrefillCase:
    hkv, d, dt = spec.num_kv_heads, spec.head_dim, spec.dtype
    B = int(ql.size)
    P = int(prefix_k.shape[0]) if shared else 0
    if shared and P % bs:
        raise ValueError("a shared prefix must fill whole blocks")
    kl = pl + ql
    if shared:
        sb = P // bs
        private = [int(math.ceil(int(kl[b]) / bs)) - sb for b in range(B)]
    else:
        sb = 0
        private = [int(math.ceil(int(kl[b]) / bs)) for b in range(B)]
    tables, nb = _allocate(_rng(perm_seed, _S_PAGING), sb, private, None, spec.free_frac, width)
    k_cache = _empty_pool(nb, bs, hkv, d, dt, poison, "k")
    v_cache = _empty_pool(nb, bs, hkv, d, dt, poison, "v")
    if shared:
        if B and P:
            pslots = _slots(tables, np.zeros(P, np.int64), np.arange(P), bs)
            _place(k_cache, pslots, prefix_k)
            _place(v_cache, pslots, prefix_v)
    else:
        seq = np.repeat(np.arange(B), pl)
        pos = np.arange(int(prefix_off[-1])) - np.repeat(prefix_off[:-1], pl)
        pslots = _slots(tables, seq, pos, bs)
        _place(k_cache, pslots, prefix_k)
        _place(v_cache, pslots, prefix_v)
    Tq = int(ql.sum())
    cu_q = np.zeros(B + 1, np.int64)
    np.cumsum(ql, out=cu_q[1:])
    cu_k = np.zeros(B + 1, np.int64)
    np.cumsum(kl, out=cu_k[1:])
    seq = np.repeat(np.arange(B), ql)
    pos = np.arange(Tq) - np.repeat(cu_q[:-1], ql) + np.repeat(pl, ql)
    new_slots = _slots(tables, seq, pos, bs).astype(np.int32)
    return PrefillCase(spec=spec, dtype=dt, num_q_heads=spec.num_q_heads, num_kv_heads=hkv,
                       head_dim=d, block_size=bs, num_blocks=nb,
                       cu_seqlens_q=cu_q.astype(np.int32), cu_seqlens_k=cu_k.astype(np.int32),
                       block_tables=tables, slot_mapping=new_slots, k_cache=k_cache,
                       v_cache=v_cache, k_new=k_new, v_new=v_new, q=q,
                       scale=np.float32(1.0 / math.sqrt(d)), prefix_lens=pl.astype(np.int32),
                       prefix_k=prefix_k, prefix_v=prefix_v, prefix_off=prefix_off,
                       shared_prefix=shared, poison=poison)


def make_prefill(spec: PrefillSpec, seed: int, block_size: Optional[int] = None,
                 perm_seed: Optional[int] = None, poison: str = "nan",
                 q_lens: Optional[Sequence[int]] = None,
                 prefix_lens: Optional[Sequence[int]] = None) -> PrefillCase:
    """Draw a varlen prefill step.  Draw order: lengths, prefix K, prefix V,
    new K, new V, Q.  With ``token_budget``, prompt lengths are drawn one at a
    time and appended while the packed total stays within the budget; the
    first draw that would overflow ends the batch.  New tokens of sequence b
    sit at positions ``prefix_lens[b] ..``; with ``shared_prefix`` every
    sequence's table starts with the same physical blocks."""
    bs = spec.block_size if block_size is None else block_size
    perm_seed = seed if perm_seed is None else perm_seed
    hq, hkv, d, dt = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    lo, hi = spec.q_len_range
    rng = _rng(seed, _S_LENGTHS)
    if q_lens is not None:
        ql = np.asarray(q_lens, np.int64)
    elif spec.q_lens is not None:
        ql = np.asarray(spec.q_lens, np.int64)
    elif spec.token_budget is not None:
        lst, tot = [], 0
        while True:
            L = int(rng.integers(lo, hi, endpoint=True))
            if tot + L > spec.token_budget:
                break
            lst.append(L)
            tot += L
        ql = np.asarray(lst, np.int64)
    else:
        ql = rng.integers(lo, hi, endpoint=True, size=spec.num_seqs)
    B = int(ql.size)
    shared = spec.shared_prefix
    if prefix_lens is not None:
        pl = np.asarray(prefix_lens, np.int64)
        shared = False
    elif spec.prefix_lens is not None:
        pl = np.asarray(spec.prefix_lens, np.int64)
        shared = False
    else:
        pl = np.full(B, spec.prefix_len, np.int64)
    if np.any(ql < 0) or np.any(pl < 0):
        raise ValueError("lengths must be non-negative")
    prefix_off = np.zeros(B + 1, np.int64)
    if shared:
        n_prefix = int(spec.prefix_len)
    else:
        np.cumsum(pl, out=prefix_off[1:])
        n_prefix = int(prefix_off[-1])
    prefix_k = _normal_rows(seed, _S_PREFIX_K, n_prefix, (hkv, d), dt)
    prefix_v = _normal_rows(seed, _S_PREFIX_V, n_prefix, (hkv, d), dt)
    Tq = int(ql.sum())
    k_new = _normal_rows(seed, _S_NEW_K, Tq, (hkv, d), dt)
    v_new = _normal_rows(seed, _S_NEW_V, Tq, (hkv, d), dt)
    q = _normal_rows(seed, _S_Q, Tq, (hq, d), dt)
    return _page_prefill(spec, ql, pl, shared, prefix_k, prefix_v, prefix_off, k_new, v_new,
                         q, bs, perm_seed, poison)


def prefill_subset(case: PrefillCase, seqs: Sequence[int], perm_seed: int = 0,
                   block_size: Optional[int] = None, table_width: int = 0) -> PrefillCase:
    """The same sequences (same content, fresh paging) alone or reordered."""
    seqs = list(seqs)
    ql = case.q_lens[seqs].astype(np.int64)
    pl = case.prefix_lens[seqs].astype(np.int64)
    cq = case.cu_seqlens_q

    def rows(a):
        parts = [a[cq[b]:cq[b + 1]] for b in seqs]
        return np.concatenate(parts) if parts else a[:0]

    if case.shared_prefix:
        pk, pv, poff = case.prefix_k, case.prefix_v, np.zeros(len(seqs) + 1, np.int64)
    else:
        po = case.prefix_off
        pk = [case.prefix_k[po[b]:po[b + 1]] for b in seqs]
        pv = [case.prefix_v[po[b]:po[b + 1]] for b in seqs]
        pk = np.concatenate(pk) if pk else case.prefix_k[:0]
        pv = np.concatenate(pv) if pv else case.prefix_v[:0]
        poff = np.zeros(len(seqs) + 1, np.int64)
        np.cumsum(pl, out=poff[1:])
    bs = case.block_size if block_size is None else block_size
    return _page_prefill(case.spec, ql, pl, case.shared_prefix, pk, pv, poff, rows(case.k_new),
                         rows(case.v_new), rows(case.q), bs, perm_seed, case.poison,
                         table_width)


def make_case(config: int, seed: Optional[int] = None, **kw):
    """Case for one of the five numbered workloads (seed defaults to the number)."""
    spec = CONFIGS[config]
    seed = config if seed is None else seed
    if isinstance(spec, DecodeSpec):
        return make_decode(spec, seed, **kw)
    return make_prefill(spec, seed, **kw)


def logical_prefix(case: PrefillCase, b: int):
    """Cached prefix rows of sequence b (shared or private), logical order."""
    if case.shared_prefix:
        return case.prefix_k, case.prefix_v
    lo, hi = case.prefix_off[b], case.prefix_off[b + 1]
    return case.prefix_k[lo:hi], case.prefix_v[lo:hi]


# ---------------------------------------------------------------- store prologue

@dataclass
class PrologueCase:
    """Raw projections of one step's new tokens plus what the store prologue
    needs: per-head norm gains, token positions, the rotary table and the
    pools (taken from an attention case, so the slots are real)."""
    q: np.ndarray            # [T, Hq, D] storage dtype
    k: np.ndarray            # [T, Hkv, D]
    v: np.ndarray            # [T, Hkv, D]
    q_weight: np.ndarray     # [D]
    k_weight: np.ndarray     # [D]
    positions: np.ndarray    # int32 [T]
    cos_sin: np.ndarray      # float32 [max_position, D]
    k_cache: np.ndarray
    v_cache: np.ndarray
    slot_mapping: np.ndarray
    dtype: str
    eps: float


def rope_table(max_position: int, head_dim: int, theta: float = 1.0e6) -> np.ndarray:
    """The rotary table a model precomputes once (an input to both sides):
    row p holds cos(p * f_i) for i < D/2, then sin(p * f_i), with
    f_i = theta^(-2i/D); float64 arithmetic, stored as float32."""
    half = head_dim // 2
    f = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * f[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_prologue(config: int, seed: int, max_position: int = 4096,
                  eps: float = 1e-6) -> PrologueCase:
    """Projections for the new tokens of attention workload ``config``: the
    same tokens, slots and pools, positions = each token's place in its
    sequence."""
    case = make_case(config)
    dt = case.dtype
    T, hkv, d = case.k_new.shape
    hq = case.num_q_heads
    rng = _rng(seed, _S_PROLOGUE)
    def draw(shape, scale=1.0, mean=0.0):
        x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale) + np.float32(mean))
        return bf16_bits(x) if dt == "bf16" else x.astype(np.float32)
    q = draw((T, hq, d), 2.0)
    k = draw((T, hkv, d), 2.0)
    v = draw((T, hkv, d))
    qw, kw = draw((d,), 0.1, 1.0), draw((d,), 0.1, 1.0)
    if hasattr(case, "context_lens"):          # decode: the new token is the last one
        pos = case.context_lens.astype(np.int64) - 1
    else:                                      # prefill: the last Lq tokens of each sequence
        pos = np.concatenate([np.arange(int(lk) - int(lq), int(lk)) for lq, lk in
                              zip(case.q_lens, case.k_lens)]) if case.num_seqs else np.zeros(0)
    pos = pos.astype(np.int32)
    if pos.size and pos.max() >= max_position:
        max_position = int(pos.max()) + 1
    return PrologueCase(q, k, v, qw, kw, pos, rope_table(max_position, d), case.k_cache,
                        case.v_cache, case.slot_mapping, dt, eps)


# --------------------------------------------------------------------------- token rows

def token_rows(tokens: Sequence[int], positions: Sequence[int], row_shape: Tuple[int, ...],
               dtype: str, seed: int, which: int) -> np.ndarray:
    """Rows that stand in for a model's per-token projections: row i is a
    N(0, 1) draw determined by (seed, which, tokens[i], positions[i]) alone,
    so a token at a given position always yields the same row, whichever
    sequence, batch or step it is computed in.  `which` picks independent
    families (say 0 = query, 1 = key, 2 = value).  Returns
    [len(tokens)] + row_shape in the storage type."""
    n = len(tokens)
    out = np.empty((n,) + tuple(row_shape), storage_np_dtype(dtype))
    m = int(np.prod(row_shape))
    for i, (t, p) in enumerate(zip(tokens, positions)):
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(_S_TOKEN_ROWS, which, int(t), int(p)))
        x = np.random.Generator(np.random.PCG64(ss)).standard_normal(m, dtype=np.float32)
        out[i] = (bf16_bits(x) if dtype == "bf16" else x).reshape(row_shape)
    return out
