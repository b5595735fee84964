"""The bf16 prefill kernel's address arithmetic, restated on the host
(``prefill_addr_model``), stays inside every buffer for the two prefill
workloads, the decode batch as one-row prompts, a mixed batch and every
ragged shape and block size the GPU tests run; each output row of each head
is stored exactly once.  Planted mistakes in the restated arithmetic are
caught.  A prefetch that reads the next item's first block-table entries
before its tile count is known strays past short sequences' blocks (and past
the table); the kernel's order (bounds first, then only existing tiles)
never does.  CPU only."""
import numpy as np
import pytest

import prefill_addr_model as m
from synth import PrefillSpec, make_case, make_prefill

RAGGED_Q = (1, 0, 37, 64, 65, 128, 200, 3)
RAGGED_P = (0, 5, 0, 64, 31, 256, 100, 700)
HEADS = [(16, 8, 128), (14, 2, 64), (8, 8, 128), (16, 4, 64), (7, 1, 128), (12, 4, 128)]
BLOCKS = [1, 16, 32, 64, 256]


def _geometry(q_lens, prefix, bs, hq=16, hkv=8, d=128, width=0, seed=0, spare=True):
    """Geometry from lengths alone: tables from a shuffled pool, `width`
    columns at least (unused entries: a spare block, or -1)."""
    ql = np.asarray(q_lens, np.int64)
    kl = ql + np.asarray(prefix, np.int64)
    need = [-(-int(k) // bs) for k in kl]
    nb = max(1, sum(need) + 1)
    ids = np.random.default_rng(seed).permutation(nb)
    mb = max(need + [1, width])
    tables = np.full((len(ql), mb), ids[-1] if spare else -1, np.int64)
    pos = 0
    for b, n in enumerate(need):
        tables[b, :n] = ids[pos:pos + n]
        pos += n
    cu_q = np.concatenate([[0], np.cumsum(ql)])
    cu_k = np.concatenate([[0], np.cumsum(kl)])
    return m.Geometry(hq, hkv, d, bs, nb, mb, int(cu_q[-1]), int(ql.max(initial=0)),
                      int(kl.max(initial=0)), cu_q, cu_k, tables)


def _check(geo):
    tot = m.check_case(geo)
    assert tot["covered_once"]
    assert tot["rows"] == sum(max(m.seq_bounds(geo, b).Lq, 0)
                              for b in range(geo.num_seqs)) * geo.num_q_heads
    return tot


@pytest.mark.parametrize("config", [4, 5])
def test_workloads_in_bounds(config):
    case = make_case(config)
    geo = m.geometry_of(case)
    assert geo.dma                          # block 256: direct-to-LDS tiles
    tot = _check(geo)
    assert tot["rows"] == case.total_q * case.num_q_heads


def test_decode_rows_and_mixed_batch_in_bounds():
    rng = np.random.default_rng(3)
    ctx = rng.integers(100, 2048, 256, endpoint=True)
    dec = _geometry(np.ones(256, np.int64), ctx - 1, 256)       # 256 one-row prompts
    assert _check(dec)["rows"] == 256 * 16
    q = np.concatenate([np.ones(256, np.int64), [512, 512, 512, 512]])
    p = np.concatenate([ctx - 1, [0, 0, 0, 0]])
    for bs in (16, 256):
        _check(_geometry(q, p, bs))


@pytest.mark.parametrize("bs", BLOCKS)
@pytest.mark.parametrize("hq,hkv,d", HEADS)
def test_ragged_shapes_in_bounds(hq, hkv, d, bs):
    spec = PrefillSpec("ragged", hq, hkv, d, "bf16", bs, q_len_range=(1, 1), q_lens=RAGGED_Q,
                       prefix_lens=RAGGED_P)
    _check(m.geometry_of(make_prefill(spec, 81)))


@pytest.mark.parametrize("bs", BLOCKS)
def test_tight_tables_and_unset_entries_in_bounds(bs):
    """Tables exactly as wide as the longest sequence, unused entries -1
    (the kernel clamps every block ID it reads into the pool)."""
    _check(_geometry(RAGGED_Q, RAGGED_P, bs, spare=False))
    _check(_geometry([3] * 1000, [0] * 1000, bs, spare=False))
    # host bounds below the lengths: the kernel clamps Lq and Lk to them
    geo = _geometry(RAGGED_Q, RAGGED_P, bs)
    geo = m.Geometry(**{**geo.__dict__, "max_seqlen_q": 40, "max_seqlen_k": 300})
    m.check_case(geo)


def test_many_sequences_in_bounds():
    rng = np.random.default_rng(7)
    _check(_geometry(rng.integers(1, 3, 2100, endpoint=True), np.zeros(2100, np.int64), 16,
                     hq=4, hkv=2, d=64))
    _check(_geometry(rng.integers(130, 300, 150, endpoint=True), np.zeros(150, np.int64), 256))


def test_planted_mistakes_are_caught(monkeypatch):
    geo = m.geometry_of(make_prefill(PrefillSpec("ragged", 16, 8, 128, "bf16", 32,
                                                 q_len_range=(1, 1), q_lens=RAGGED_Q,
                                                 prefix_lens=RAGGED_P), 81))
    # one tile too many per item: its descriptor would start past the keys
    real = m.n_tiles
    monkeypatch.setattr(m, "n_tiles", lambda g, qt, bd: real(g, qt, bd) + 1)
    with pytest.raises(m.AddressError):
        m.check_case(geo)
    monkeypatch.setattr(m, "n_tiles", real)
    # dropping the clamp of Lk to the table's width
    narrow = m.Geometry(**{**geo.__dict__, "max_blocks_per_seq": 2,
                           "tables": geo.tables[:, :2]})
    m.check_case(narrow)                                     # clamped: in bounds
    real_bounds = m.seq_bounds

    def unclamped(g, b):
        bd = real_bounds(g, b)
        kl = int(g.cu_k[b + 1] - g.cu_k[b])
        return m.Bounds(bd.q_start, bd.Lq, kl if bd.Lq > 0 else bd.Lk)

    monkeypatch.setattr(m, "seq_bounds", unclamped)
    with pytest.raises(m.AddressError):
        m.check_case(narrow)
    monkeypatch.setattr(m, "seq_bounds", real_bounds)
    # an item of one head too many
    with pytest.raises(m.AddressError):
        m.item_accesses(geo, 0, 0, geo.num_kv_heads)


def _stray(geo, reads):
    out = []
    for it in m.items(geo):
        out += m.stray_reads(geo, reads(geo, it))
    return out


@pytest.mark.parametrize("bs", [32, 64])
def test_early_block_reads_stray_guarded_do_not(bs):
    geo = _geometry(RAGGED_Q, RAGGED_P, bs)
    early = _stray(geo, m.early_block_reads)
    assert any("past its" in s for s in early)              # a one-token prompt
    assert _stray(geo, m.guarded_block_reads) == []
    # many short prompts, table one block wide: the last one reads past the table
    short = _geometry([5] * 1000, [0] * 1000, bs)
    early = _stray(short, m.early_block_reads)
    assert any("past the end of the table" in s for s in early)
    assert _stray(short, m.guarded_block_reads) == []


@pytest.mark.parametrize("config", [4, 5])
def test_guarded_block_reads_on_workloads(config):
    geo = m.geometry_of(make_case(config))
    assert _stray(geo, m.guarded_block_reads) == []
    # at block 256 the first three tiles always sit in block 0: the early
    # order reads nothing stray on these workloads
    assert _stray(geo, m.early_block_reads) == []


def test_direct_to_lds_path_needs_a_32_bit_block_stride():
    """Block sizes whose byte stride would not fit in 32 bits take the
    register loader (the launcher's test, restated by the model)."""
    z = np.zeros(2, np.int64)
    t = np.zeros((1, 1), np.int64)
    ok = m.Geometry(16, 8, 128, 1 << 20, 1, 1, 1, 1, 1, z, z, t)   # 2 GiB per block
    big = m.Geometry(16, 8, 128, 1 << 21, 1, 1, 1, 1, 1, z, z, t)  # 4 GiB per block
    assert ok.dma and not big.dma
