"""Plain Python model of the host block manager (the bookkeeping that yields
the kernels' block tables and slot mapping).

TEST INFRASTRUCTURE ONLY (the same rule as the attention oracle): only the
tests may use it, and it shares no code with the C++ manager in libpa.

What it models, and where the pages say so:

* a fixed pool of equal blocks handed out from a free list, first in first
  out ("mini-vLLM", features list: constant-time block hand-out from a pool
  fixed at start-up; every sequence keeps its own table of blocks);
* full blocks registered by their content so that a sequence beginning with
  the same full blocks shares them, with reference counts (smzdm Nano-vLLM
  walk-through, scheduling and memory: the shared system prompt is reused;
  "nano-vLLM Part 4", comparison table: an exact full-block prefix cache);
  the key here is the exact tuple of every token up to the end of the block,
  since a block's K/V depends on all earlier tokens;
* a block whose count drops to zero returns to the free list but stays
  registered until the free list hands it out for new content, so a
  preempted sequence allocated again finds its blocks (smzdm walk-through,
  scheduling and memory; "mini-vLLM": preemption hands back every block);
* a prompt whose blocks are all cached still recomputes its last token
  (a step needs a query row); the partial last block is never shared;
* a decode token that opens a block takes a fresh one; a token that fills a
  block registers it.

Pins (CPU suite): every block comes back once all sequences are freed;
a shared system prompt is cached; blocks of live sequences are shared only
when their token prefixes are identical; a freed-and-reallocated sequence
finds all its full blocks while they are untouched; plus the C++ manager's
outputs equal this model's, operation by operation, on random workloads.
"""
from __future__ import annotations

from collections import OrderedDict


class NoMemory(Exception):
    pass


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.bs, self.num_blocks = block_size, num_blocks
        self.free = OrderedDict((b, None) for b in range(num_blocks))   # FIFO free list
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks          # registered prefix of each block
        self.registry = {}                      # prefix tuple -> block
        self.seqs = {}                          # id -> dict(tokens, blocks, cached)

    def num_free(self) -> int:
        return len(self.free)

    def _fresh(self) -> int:
        b, _ = self.free.popitem(last=False)
        if self.key[b] is not None:
            if self.registry.get(self.key[b]) == b:
                del self.registry[self.key[b]]
            self.key[b] = None
        self.ref[b] = 1
        return b

    def _register(self, b: int, prefix: tuple) -> None:
        self.key[b] = prefix
        self.registry[prefix] = b

    def allocate(self, sid, tokens) -> int:
        tokens = [int(t) for t in tokens]
        if sid in self.seqs or not tokens:
            raise ValueError("bad allocate")
        bs, n = self.bs, len(tokens)
        nblocks = -(-n // bs)
        hits = []
        for i in range(n // bs):
            b = self.registry.get(tuple(tokens[:(i + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        free_after = len(self.free) - sum(1 for b in hits if b in self.free)
        if nblocks - len(hits) > free_after:
            raise NoMemory()
        blocks, cached = [], 0
        for i in range(nblocks):
            if i < len(hits):
                b = hits[i]
                if b in self.free:
                    del self.free[b]
                    self.ref[b] = 1
                else:
                    self.ref[b] += 1
                cached += bs
            else:
                b = self._fresh()
                if (i + 1) * bs <= n:
                    self._register(b, tuple(tokens[:(i + 1) * bs]))
            blocks.append(b)
        cached = min(cached, n - 1)
        self.seqs[sid] = {"tokens": tokens, "blocks": blocks, "cached": cached}
        return cached

    def append(self, sid, token) -> int:
        s = self.seqs[sid]
        bs, n = self.bs, len(s["tokens"])
        if n % bs == 0:
            if not self.free:
                raise NoMemory()
            s["blocks"].append(self._fresh())
        s["tokens"].append(int(token))
        b = s["blocks"][n // bs]
        if (n + 1) % bs == 0:
            self._register(b, tuple(s["tokens"][:n + 1]))
        return b * bs + n % bs

    def release(self, sid) -> None:
        s = self.seqs.pop(sid)
        for b in reversed(s["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free[b] = None

    def block_table(self, sid):
        return list(self.seqs[sid]["blocks"])

    def slots(self, sid, first, count):
        s = self.seqs[sid]
        return [s["blocks"][j // self.bs] * self.bs + j % self.bs for j in range(first, first + count)]
