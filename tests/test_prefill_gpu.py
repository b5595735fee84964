"""pa_prefill_varlen on the GPU against the fp64 oracle, plus invariants.

bf16 runs on the matrix cores; fp32 on the vector path.  Parity bar: fp32
max-abs <= 1e-5; bf16 max-abs <= 2e-2 and mean-abs <= 2e-3 over every output
element.  The two numbered prefill workloads run at full size.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import assert_close, bits, dev, f64, run_decode, run_prefill, say
from synth import DecodeSpec, PrefillSpec, make_case, make_decode, make_prefill, prefill_subset

pytestmark = pytest.mark.gpu


def _oracle(case):
    kc, vc = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new,
                             case.slot_mapping)
    return oracle.prefill_varlen(case.q, kc, vc, case.block_tables, case.cu_seqlens_q,
                                 case.cu_seqlens_k, case.scale, case.dtype)


@pytest.mark.parametrize("config", [4, 5])
def test_prefill_configs(config):
    case = make_case(config)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), case.dtype, f"config {config}")


SHAPES = [
    # (Hq, Hkv, D, dtype)
    (16, 8, 128, "bf16"), (14, 2, 64, "bf16"), (8, 8, 128, "bf16"), (16, 4, 64, "bf16"),
    (7, 1, 128, "bf16"), (12, 4, 128, "bf16"), (4, 2, 64, "f32"), (16, 8, 128, "f32"),
    (6, 2, 64, "f32"),
]


@pytest.mark.parametrize("hq,hkv,d,dtype", SHAPES)
@pytest.mark.parametrize("bs", [1, 16, 32, 64, 256])
def test_prefill_shapes_ragged(hq, hkv, d, dtype, bs):
    """Ragged tails, empty and one-token prompts, prefixes that do and do not
    end on a tile or block boundary."""
    q_lens = (1, 0, 37, 64, 65, 128, 200, 3)
    prefix = (0, 5, 0, 64, 31, 256, 100, 700)
    spec = PrefillSpec(f"pre-{hq}-{hkv}-{d}-{dtype}", hq, hkv, d, dtype, bs, q_len_range=(1, 1),
                       q_lens=q_lens, prefix_lens=prefix)
    case = make_prefill(spec, 81)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), dtype, spec.name + f" bs{bs}")


@pytest.mark.parametrize("poison", ["big", "zero"])
def test_prefill_poison(poison):
    spec = PrefillSpec("pre-poison", 16, 8, 128, "bf16", 16, q_len_range=(1, 1),
                       q_lens=(5, 70, 129), prefix_lens=(3, 0, 64))
    case = make_prefill(spec, 82, poison=poison)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), "bf16", f"prefill poison {poison}")


@pytest.mark.parametrize("config", [4, 5])
def test_prefill_work_counter_bitwise(config):
    """Query tiles dealt through the work counter (whichever workgroup is
    free) or in the fixed snake give the same bits, and every call leaves the
    counter at zero."""
    import torch
    case = make_case(config)
    fixed, _, _ = run_prefill(case, workspace=False)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda:0")
    for rep in range(3):
        dealt, _, _ = run_prefill(case, workspace=ws)
        assert np.array_equal(bits(dealt), bits(fixed)), f"config {config} call {rep}"
        assert int(ws.count_nonzero()) == 0, "the work counter must come back to zero"


def test_prefill_many_sequences_deals_bitwise():
    """150 sequences of two to five query tiles (8 KV heads, block 256): the
    work-counter launch deals each KV head's tiles within one group of
    workgroups and walks several 64-sequence chunks per group.  It must give
    the fixed deal's bits and leave every counter at zero; sampled sequences
    run alone match the oracle and their batched rows."""
    import torch
    spec = PrefillSpec("pre-many", 16, 8, 128, "bf16", 256, q_len_range=(130, 300),
                       num_seqs=150, prefix_len=40)
    case = make_prefill(spec, 84)
    fixed, _, _ = run_prefill(case, workspace=False)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda:0")
    for rep in range(2):
        dealt, _, _ = run_prefill(case, workspace=ws)
        assert np.array_equal(bits(dealt), bits(fixed)), f"call {rep}"
        assert int(ws.count_nonzero()) == 0, "the work counters must come back to zero"
    cq = case.cu_seqlens_q
    for b in (0, 77, 149):
        sub = prefill_subset(case, [b], perm_seed=b + 1)
        alone = run_prefill(sub)[0]
        assert np.array_equal(bits(alone), bits(fixed)[cq[b]:cq[b + 1]]), b
        assert_close(f64(alone), _oracle(sub), "bf16", f"pre-many seq {b}")


def test_prefill_beyond_persistent_batch():
    """2100 one- to three-token prompts: more sequences than the persistent
    launch keeps counts for, so one workgroup per item; against the oracle."""
    spec = PrefillSpec("pre-2100", 4, 2, 64, "bf16", 16, q_len_range=(1, 3), num_seqs=2100,
                       prefix_len=5)
    case = make_prefill(spec, 85)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), "bf16", spec.name)


def test_prefill_invariance_bitwise():
    spec = PrefillSpec("pre-inv", 16, 8, 128, "bf16", 16, q_len_range=(1, 1),
                       q_lens=(40, 130, 1, 77), prefix_lens=(0, 20, 256, 5))
    ref = bits(run_prefill(make_prefill(spec, 83))[0])
    for bs in (1, 4, 32, 64, 256):
        assert np.array_equal(bits(run_prefill(make_prefill(spec, 83, block_size=bs))[0]), ref)
    assert np.array_equal(bits(run_prefill(make_prefill(spec, 83, perm_seed=7))[0]), ref)
    case = make_prefill(spec, 83)
    cq = case.cu_seqlens_q
    for b in range(case.num_seqs):
        alone = run_prefill(prefill_subset(case, [b], perm_seed=b + 3))[0]
        assert np.array_equal(bits(alone), ref[cq[b]:cq[b + 1]]), b


def test_prefix_prefill_sampled_alone():
    """Shared-prefix workload: sampled sequences alone equal their batched rows."""
    case = make_case(5)
    ref = bits(run_prefill(case)[0])
    cq = case.cu_seqlens_q
    for b in (0, 31, 63):
        alone = run_prefill(prefill_subset(case, [b], perm_seed=11))[0]
        assert np.array_equal(bits(alone), ref[cq[b]:cq[b + 1]])


def test_prefill_rows_match_decode_fp32():
    """Prefill row i is a decode over Lk - Lq + i + 1 keys (two different
    kernels, so agreement is to the fp32 tolerance)."""
    spec = PrefillSpec("pre-vs-dec", 8, 2, 64, "f32", 16, q_len_range=(1, 1),
                       q_lens=(9, 20), prefix_lens=(30, 0))
    case = make_prefill(spec, 84)
    out, kc, vc = run_prefill(case)
    out = f64(out)
    import torch
    import paged_kv_cache_85_amd as pa
    bt = dev(case.block_tables)
    for b in range(case.num_seqs):
        q0, q1 = case.cu_seqlens_q[b], case.cu_seqlens_q[b + 1]
        lk = case.cu_seqlens_k[b + 1] - case.cu_seqlens_k[b]
        lq = q1 - q0
        rows = dev(case.q[q0:q1])
        lens = dev(np.asarray([lk - lq + i + 1 for i in range(lq)], np.int32))
        dec = torch.empty_like(rows)
        bt_rows = bt[b:b + 1].repeat(lq, 1).contiguous()
        pa.pa_decode(dec, rows, kc, vc, bt_rows, lens, int(lk), float(case.scale))
        torch.cuda.synchronize()
        assert np.abs(f64(dec) - out[q0:q1]).max() <= 2e-6


def test_prefill_empty_is_noop():
    import torch
    import paged_kv_cache_85_amd as pa
    z = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    pool = torch.zeros((4, 16, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros((2, 1), dtype=torch.int32, device="cuda:0")
    cu = torch.zeros((3,), dtype=torch.int32, device="cuda:0")
    pa.pa_prefill_varlen(z, z, pool, pool, bt, cu, cu, 0, 0, 0.125)


def test_prefill_block_stride_past_32_bits_matches_small_blocks():
    """A 4 GiB block (2^24 rows of 2 heads x 64 bf16) has a byte stride that
    the direct-to-LDS loads do not hold in 32 bits, so the call gathers its
    tiles row by row; the output equals that of a pool of 256-token blocks bit
    for bit (both loaders fill the same LDS layout)."""
    import math

    import torch

    import paged_kv_cache_85_amd as pa
    rng = np.random.default_rng(11)
    L, hq, hkv, d = 150, 4, 2, 64

    def bf(shape):
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(
            torch.bfloat16).to("cuda:0")

    q, k, v = bf((L, hq, d)), bf((L, hkv, d)), bf((L, hkv, d))
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda:0")
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda:0")
    slots = torch.arange(L, dtype=torch.int32, device="cuda:0")
    outs = []
    for bs in (256, 1 << 24):
        say(f"block_size {bs}: pools of {bs * hkv * d * 2 / 2**30:.3g} GiB each")
        kc = torch.empty((1, bs, hkv, d), dtype=torch.bfloat16, device="cuda:0")
        vc = torch.empty_like(kc)
        pa.pa_store_kv(k, v, kc, vc, slots)
        out = torch.empty_like(q)
        pa.pa_prefill_varlen(out, q, kc, vc, bt, cu, cu, L, L, 1.0 / math.sqrt(d))
        torch.cuda.synchronize()
        outs.append(bits(out))
        del kc, vc
        torch.cuda.empty_cache()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("bs", [256, 16])
def test_prefill_long_prompts_sampled(bs):
    """Long items: a 12,000-token prompt (375 key tiles for its last query
    tile), a 3,000-token one and a short one behind a 500-token cached
    prefix.  The whole call runs on the GPU; 96 sampled rows are checked
    against the oracle, each as attention over its own visible keys."""
    spec = PrefillSpec(f"pre-long-{bs}", 8, 4, 128, "bf16", bs, q_len_range=(1, 1),
                       q_lens=(12000, 37, 3000), prefix_lens=(0, 500, 0))
    case = make_prefill(spec, 61)
    out, _, _ = run_prefill(case)
    out = f64(out)
    kc, vc = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new,
                             case.slot_mapping)
    rng = np.random.default_rng(5)
    for b in range(case.num_seqs):
        q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        lk = int(case.cu_seqlens_k[b + 1] - case.cu_seqlens_k[b])
        lq = q1 - q0
        rows = np.unique(np.concatenate([[0, lq - 1], rng.integers(0, lq, 30)]))
        lens = np.asarray([lk - lq + i + 1 for i in rows], np.int32)
        bt = np.repeat(case.block_tables[b:b + 1], len(rows), axis=0)
        ref = oracle.decode(case.q[q0 + rows], kc, vc, bt, lens, case.scale, case.dtype)
        assert_close(out[q0 + rows], ref, "bf16", f"{spec.name} sequence {b}")
