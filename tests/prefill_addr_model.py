"""Host model of the bf16 prefill kernel's address arithmetic, with bounds
checks (test infrastructure; no GPU).

It restates, in Python, every index and byte range the kernel in
``paged_kv_cache_85_amd/csrc/prefill.hip`` computes from the call's
arguments: the per-sequence bounds read from cu_seqlens_q / cu_seqlens_k
(with the kernel's clamps), the query-tile items, the block-table entry
read for each key/value tile, the buffer descriptor of each direct-to-LDS
tile request (base and byte count), the rows the register loader gathers
for other block sizes, the Q rows loaded and the output rows stored, and the
LDS stage each request fills.  ``check_case`` walks every item of a call and
raises ``AddressError`` at the first access outside its buffer.

It also models one prefetch schedule that is not in the kernel: the next
item's bounds and the block-table entries of its first ring tiles read in
one batch, before the item's tile count is known (``early_block_reads``).
The kernel reads a tile's block only once that tile is known to exist
(``guarded_block_reads``).

The constants mirror the kernel's compile-time choices: 32-key tiles, a
ring of three stages, four waves of 32 query rows, heads per wave from the
query-group size.
"""
from dataclasses import dataclass
from typing import Iterator, List, Sequence, Tuple

import numpy as np

BN = 32      # keys per tile
NST = 3      # tile stages in LDS
WAVES = 4    # waves per workgroup, 32 query rows each
ELEM = 2     # bf16 bytes


class AddressError(AssertionError):
    pass


@dataclass(frozen=True)
class Geometry:
    """The arguments of one pa_prefill_varlen call that address memory."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    total_q: int
    max_seqlen_q: int
    max_seqlen_k: int
    cu_q: np.ndarray          # int [B + 1]
    cu_k: np.ndarray          # int [B + 1]
    tables: np.ndarray        # int [B, max_blocks_per_seq]

    @property
    def num_seqs(self) -> int:
        return int(self.cu_q.shape[0]) - 1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def hpw(self) -> int:
        g = self.group
        return 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1

    @property
    def bmq(self) -> int:
        return 32 * (WAVES // self.hpw)

    @property
    def bs_log2(self) -> int:
        bs = self.block_size
        return bs.bit_length() - 1 if bs & (bs - 1) == 0 else -1

    @property
    def dma(self) -> bool:
        # Direct-to-LDS tiles need whole tiles inside a block, and the kernel
        # keeps a block's byte stride in 32 bits.
        return (self.bs_log2 >= 0 and self.block_size >= BN and
                self.block_size * self.row_bytes < (1 << 32))

    @property
    def row_bytes(self) -> int:
        return self.num_kv_heads * self.head_dim * ELEM

    @property
    def pool_bytes(self) -> int:
        return self.num_blocks * self.block_size * self.row_bytes


def geometry_of(case) -> Geometry:
    """Geometry of a synthetic prefill case (``synth.PrefillCase``)."""
    return Geometry(case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size,
                    case.num_blocks, case.max_blocks_per_seq, case.total_q, case.max_seqlen_q,
                    case.max_seqlen_k, case.cu_seqlens_q.astype(np.int64),
                    case.cu_seqlens_k.astype(np.int64), case.block_tables.astype(np.int64))


@dataclass(frozen=True)
class Bounds:
    q_start: int
    Lq: int
    Lk: int

    @property
    def delta(self) -> int:
        return self.Lk - self.Lq


def seq_bounds(geo: Geometry, b: int) -> Bounds:
    """A sequence's clamped bounds, as the kernel derives them (Lq <= 0 when
    the sequence contributes no rows)."""
    if not 0 <= b < geo.num_seqs:
        raise AddressError(f"sequence index {b} outside [0, {geo.num_seqs})")
    qs, qe = int(geo.cu_q[b]), int(geo.cu_q[b + 1])
    kl = int(geo.cu_k[b + 1] - geo.cu_k[b])
    if qs < 0 or qs >= geo.total_q:
        return Bounds(qs, 0, 0)
    Lk = min(kl, geo.max_seqlen_k, geo.max_blocks_per_seq * geo.block_size)
    Lq = min(qe - qs, geo.max_seqlen_q, Lk, geo.total_q - qs)
    return Bounds(qs, Lq, Lk)


def n_tiles(geo: Geometry, qt: int, bd: Bounds) -> int:
    kmax_wg = bd.delta + min(qt * geo.bmq + geo.bmq, bd.Lq) - 1
    return kmax_wg // BN + 1


def items(geo: Geometry) -> Iterator[Tuple[int, int, int]]:
    """Non-empty (query tile, sequence, KV head / head chunk) items, heaviest
    first: the order the persistent kernel walks."""
    inner = geo.num_kv_heads * (geo.group // geo.hpw)
    nq = []
    for b in range(geo.num_seqs):
        bd = seq_bounds(geo, b)
        nq.append(-(-bd.Lq // geo.bmq) if bd.Lq > 0 else 0)
    n_qt = -(-geo.max_seqlen_q // geo.bmq)
    for qt in range(n_qt - 1, -1, -1):
        for b in range(geo.num_seqs):
            if nq[b] > qt:
                for gh in range(inner):
                    yield qt, b, gh


def _table_entry(geo: Geometry, b: int, idx: int) -> int:
    if not 0 <= idx < geo.max_blocks_per_seq:
        raise AddressError(f"block-table index {idx} of sequence {b} outside its row "
                           f"of {geo.max_blocks_per_seq}")
    blk = int(geo.tables[b, idx])
    return min(max(blk, 0), geo.num_blocks - 1)        # the kernel clamps into the pool


def tile_request(geo: Geometry, b: int, g: int, kt: int, bd: Bounds) -> Tuple[int, int]:
    """Byte range [lo, hi) of the pool a direct-to-LDS request of tile kt
    reads: descriptor base at the tile's first row (head g), byte count
    min(BN, Lk - t0) rows; lanes past the count read zero."""
    t0 = kt * BN
    blk = _table_entry(geo, b, t0 >> geo.bs_log2)
    rows = min(BN, bd.Lk - t0)
    if rows < 1:
        raise AddressError(f"tile {kt} of sequence {b} starts past its {bd.Lk} keys "
                           f"(descriptor byte count {rows} rows)")
    off = t0 & (geo.block_size - 1)
    if off + rows > geo.block_size:
        raise AddressError(f"tile {kt} of sequence {b} leaves its block")
    lo = ((blk * geo.block_size + off) * geo.num_kv_heads + g) * geo.head_dim * ELEM
    # The kernel's form of the same base: the head's row in the pool, plus
    # block x (32-bit block stride) and row-in-block x row bytes, both
    # products in unsigned 32-bit arithmetic.
    blk_bytes = geo.block_size * geo.row_bytes
    in_blk = off * geo.row_bytes
    if not (blk_bytes < (1 << 32) and in_blk < (1 << 32)):
        raise AddressError(f"32-bit stride overflow (block bytes {blk_bytes}, row offset {in_blk})")
    kernel_lo = g * geo.head_dim * ELEM + blk * blk_bytes + in_blk
    if kernel_lo != lo:
        raise AddressError(f"descriptor base {kernel_lo} differs from the slot formula's {lo}")
    hi = lo + (rows - 1) * geo.row_bytes + geo.head_dim * ELEM
    return lo, hi


def gathered_rows(geo: Geometry, b: int, g: int, kt: int, bd: Bounds) -> Tuple[int, int]:
    """Byte range the register loader touches for tile kt (one block-table
    lookup per key row; rows past Lk are not read)."""
    lo_all, hi_all = None, None
    for j in range(kt * BN, min(kt * BN + BN, bd.Lk)):
        idx = j >> geo.bs_log2 if geo.bs_log2 >= 0 else j // geo.block_size
        blk = _table_entry(geo, b, idx)
        slot = blk * geo.block_size + j % geo.block_size
        lo = (slot * geo.num_kv_heads + g) * geo.head_dim * ELEM
        hi = lo + geo.head_dim * ELEM
        lo_all = lo if lo_all is None else min(lo_all, lo)
        hi_all = hi if hi_all is None else max(hi_all, hi)
    if lo_all is None:
        raise AddressError(f"tile {kt} of sequence {b} holds no key")
    return lo_all, hi_all


def check_lds_layout(geo: Geometry) -> None:
    """Every wave's 1 KiB request slices tile their stage's K (then V) half
    exactly; the LDS byte addresses the kernel hands the loads (stage base +
    wave slice, V half after the K half) cover the NST stages once."""
    cpr = geo.head_dim // 8
    ni = BN * cpr // 256
    half = BN * geo.head_dim
    covered = np.zeros(half, np.int32)
    for w in range(WAVES):
        for i in range(ni):
            lo = (w * ni + i) * 512
            if lo < 0 or lo + 512 > half:
                raise AddressError(f"LDS slice {lo} of wave {w} outside the stage half")
            covered[lo:lo + 512] += 1
    stage_bytes = 2 * half * ELEM
    lds = np.zeros(NST * stage_bytes, np.int32)
    for stage in range(NST):
        for w in range(WAVES):
            dk = stage * stage_bytes + w * ni * 1024
            dv = dk + half * ELEM
            for i in range(ni):
                for a in (dk + i * 1024, dv + i * 1024):
                    if a < 0 or a + 1024 > lds.size:
                        raise AddressError(f"LDS byte address {a} outside the stages")
                    lds[a:a + 1024] += 1
    if not np.all(lds == 1):
        raise AddressError("LDS byte addresses do not cover the stages exactly once")
    if not np.all(covered == 1):
        raise AddressError("the request slices do not tile the stage half exactly")


def item_accesses(geo: Geometry, qt: int, b: int, gh: int, seen=None) -> dict:
    """Check every access of one item; returns a small tally.  With `seen`
    (bool [total_q, num_q_heads]) also checks that no output row of a head
    is stored twice."""
    hchunks = geo.group // geo.hpw
    g, hc = gh // hchunks, gh % hchunks
    if not 0 <= g < geo.num_kv_heads:
        raise AddressError(f"KV head {g}")
    bd = seq_bounds(geo, b)
    if bd.Lq <= 0 or qt * geo.bmq >= bd.Lq:
        return {"tiles": 0, "rows": 0}
    nt = n_tiles(geo, qt, bd)
    if nt < 1 or (nt - 1) * BN >= bd.Lk:
        raise AddressError(f"item ({qt}, {b}) spans {nt} tiles over {bd.Lk} keys")
    for kt in range(nt):
        lo, hi = (tile_request if geo.dma else gathered_rows)(geo, b, g, kt, bd)
        if lo < 0 or hi > geo.pool_bytes:
            raise AddressError(f"tile {kt} of sequence {b}: bytes [{lo}, {hi}) outside "
                               f"the {geo.pool_bytes}-byte pool")
    rows = 0
    wph = WAVES // geo.hpw
    for w in range(WAVES):
        h = g * geo.group + hc * geo.hpw + w // wph
        if not 0 <= h < geo.num_q_heads:
            raise AddressError(f"query head {h}")
        row0 = qt * geo.bmq + (w % wph) * 32
        for r in range(row0, min(row0 + 32, bd.Lq)):
            t = bd.q_start + r
            if not 0 <= t < geo.total_q:
                raise AddressError(f"query row {t} outside [0, {geo.total_q})")
            if seen is not None:
                if seen[t, h]:
                    raise AddressError(f"output row {t} of head {h} stored twice")
                seen[t, h] = True
            rows += 1
    return {"tiles": nt, "rows": rows}


def check_case(geo: Geometry) -> dict:
    """Check every item of a call; returns totals (items, tile requests,
    query-row loads) and whether every row of every sequence's clamped query
    range is stored for every head exactly once."""
    check_lds_layout(geo)
    seen = np.zeros((geo.total_q, geo.num_q_heads), bool)
    tot = {"items": 0, "tiles": 0, "rows": 0}
    for qt, b, gh in items(geo):
        t = item_accesses(geo, qt, b, gh, seen)
        tot["items"] += 1
        tot["tiles"] += t["tiles"]
        tot["rows"] += t["rows"]
    want = np.zeros_like(seen)
    for b in range(geo.num_seqs):
        bd = seq_bounds(geo, b)
        if bd.Lq > 0:
            want[bd.q_start:bd.q_start + bd.Lq] = True
    tot["covered_once"] = bool(np.array_equal(seen, want))
    return tot


# --------------------------------------------------------------------------
# Cross-item prefetch: which block-table entries of the next item are read.

def sequence_blocks(geo: Geometry, b: int) -> int:
    """Blocks that hold the sequence's keys (the valid part of its row)."""
    bd = seq_bounds(geo, b)
    return -(-max(bd.Lk, 0) // geo.block_size)


def early_block_reads(geo: Geometry, item: Tuple[int, int, int]) -> List[Tuple[int, int]]:
    """(sequence, table index) of the next item's first NST tiles, read in
    the same batch as its bounds: the tile count is not known yet."""
    _, b, _ = item
    return [(b, (t * BN) >> geo.bs_log2) for t in range(NST)]


def guarded_block_reads(geo: Geometry, item: Tuple[int, int, int]) -> List[Tuple[int, int]]:
    """The kernel's order: bounds first, then only tiles t < n_tiles."""
    qt, b, _ = item
    bd = seq_bounds(geo, b)
    nt = n_tiles(geo, qt, bd)
    return [(b, (t * BN) >> geo.bs_log2) for t in range(min(NST, nt))]


def stray_reads(geo: Geometry, reads: Sequence[Tuple[int, int]]) -> List[str]:
    """Reads past the sequence's own blocks, and past the whole table."""
    bad = []
    for b, idx in reads:
        flat = b * geo.max_blocks_per_seq + idx
        if flat >= geo.num_seqs * geo.max_blocks_per_seq:
            bad.append(f"sequence {b}: table index {idx} past the end of the table")
        elif idx >= sequence_blocks(geo, b):
            bad.append(f"sequence {b}: table index {idx} past its "
                       f"{sequence_blocks(geo, b)} block(s)")
    return bad
