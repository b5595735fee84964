"""Decode steps replayed from a captured HIP graph (launch overhead paid once).

A decode step of a small batch is short enough for launch overhead to matter
(the smzdm Nano-vLLM walk-through, GPU execution: decode runs from captured
graphs at bucketed batch sizes; "nano-vLLM Part 4", section 3).  DecodeGraph
captures pa_store_kv + pa_decode once for a fixed bucket of sequences on
static buffers; each call copies the step's inputs into those buffers and
replays.  Rows past the real batch are padding: slot -1 (the store skips
them) and context length 1 over the first real row's table, and their output
is dropped.  Every launch is one of libpa's kernels; this module only owns
buffers and replays.
"""
from __future__ import annotations

from .binding import pa_decode, pa_decode_workspace_bytes, pa_store_kv


def bucket_size(n: int) -> int:
    """Graph bucket for a batch of n sequences: powers of two up to 16, then
    multiples of 16."""
    if n <= 0:
        raise ValueError("empty batch")
    if n <= 16:
        b = 1
        while b < n:
            b *= 2
        return b
    return (n + 15) // 16 * 16


class DecodeGraph:
    """Store + decode for batches of up to ``max_seqs`` sequences, captured once.

    k_cache, v_cache: the pools [NB, BS, Hkv, D] (captured by address: the
    graph always reads and writes these two tensors).
    """

    def __init__(self, k_cache, v_cache, num_q_heads: int, max_seqs: int,
                 max_blocks_per_seq: int, max_context_len: int, scale: float):
        import torch
        nb, bs, hkv, d = k_cache.shape
        dev = k_cache.device
        self.k_cache, self.v_cache = k_cache, v_cache
        self.max_seqs, self.max_context_len, self.scale = max_seqs, max_context_len, scale
        self.q = torch.zeros(max_seqs, num_q_heads, d, dtype=k_cache.dtype, device=dev)
        self.k_new = torch.zeros(max_seqs, hkv, d, dtype=k_cache.dtype, device=dev)
        self.v_new = torch.zeros_like(self.k_new)
        self.slots = torch.full((max_seqs,), -1, dtype=torch.int32, device=dev)
        self.lens = torch.ones(max_seqs, dtype=torch.int32, device=dev)
        self.tables = torch.zeros(max_seqs, max_blocks_per_seq, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        n = pa_decode_workspace_bytes(max_seqs, num_q_heads, d, max_context_len)
        self.workspace = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
        # One eager pass first (the library caches its occupancy queries on
        # the first launch, outside the capture), then the capture.
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            self._step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step()

    def _step(self) -> None:
        pa_store_kv(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots)
        pa_decode(self.out, self.q, self.k_cache, self.v_cache, self.tables, self.lens,
                  self.max_context_len, self.scale, workspace=self.workspace)

    def __call__(self, q, k_new, v_new, slot_mapping, context_lens, block_tables):
        """One decode step for n <= max_seqs sequences; returns out[:n] (a view
        of the graph's output buffer, overwritten by the next call)."""
        n = q.shape[0]
        if n > self.max_seqs or block_tables.shape[1] > self.tables.shape[1]:
            raise ValueError("batch larger than the captured bucket")
        self.q[:n].copy_(q)
        self.k_new[:n].copy_(k_new)
        self.v_new[:n].copy_(v_new)
        self.slots[:n].copy_(slot_mapping)
        self.slots[n:].fill_(-1)
        self.lens[:n].copy_(context_lens)
        self.lens[n:].fill_(1)
        w = block_tables.shape[1]
        self.tables[:n, :w].copy_(block_tables)
        self.tables[n:, :w].copy_(block_tables[:1].expand(self.max_seqs - n, w))
        self.graph.replay()
        return self.out[:n]
