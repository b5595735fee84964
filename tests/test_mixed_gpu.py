"""Mixed batches: decode rows (one new token over a long cached context) and
prompts (with or without a cached prefix) served by one pa_prefill_varlen
launch, against the fp64 oracle.

A decode row is a varlen sequence with Lq = 1 and Lk = its context length, so
the same call covers both phases ("mini-vLLM", project summary: a decode row
is one new query per sequence over its stored history, and a prefill packs
several prompts whose rows see only earlier positions of their own prompt).  Parity bar as elsewhere: bf16 max-abs <= 2e-2 and mean-abs <=
2e-3, fp32 max-abs <= 1e-5.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import assert_close, bits, f64, run_prefill
from synth import PrefillSpec, make_prefill, prefill_subset

pytestmark = pytest.mark.gpu


def _oracle(case):
    kc, vc = oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new,
                             case.slot_mapping)
    return oracle.prefill_varlen(case.q, kc, vc, case.block_tables, case.cu_seqlens_q,
                                 case.cu_seqlens_k, case.scale, case.dtype)


def _mixed_lengths(n_decode, seed):
    """n_decode decode rows with contexts in [100, 2048], with three prompts
    (one plain, two with a cached prefix) placed among them."""
    rng = np.random.default_rng(seed)
    q = [1] * n_decode
    pre = [int(x) - 1 for x in rng.integers(100, 2048, n_decode, endpoint=True)]
    for pos, (lq, lp) in zip((0, n_decode // 2, n_decode), ((300, 0), (64, 500), (129, 77))):
        q.insert(pos, lq)
        pre.insert(pos, lp)
    return tuple(q), tuple(pre)


@pytest.mark.parametrize("bs", [16, 256])
def test_mixed_batch_bf16(bs):
    q, pre = _mixed_lengths(40, 7)
    spec = PrefillSpec("mixed-qwen3", 16, 8, 128, "bf16", bs, q_len_range=(1, 1),
                       q_lens=q, prefix_lens=pre)
    case = make_prefill(spec, 91)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), "bf16", f"mixed bf16 bs{bs}")


def test_mixed_batch_fp32():
    q, pre = _mixed_lengths(12, 8)
    spec = PrefillSpec("mixed-f32", 8, 2, 64, "f32", 16, q_len_range=(1, 1),
                       q_lens=q, prefix_lens=pre)
    case = make_prefill(spec, 92)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), "f32", "mixed fp32")


def test_mixed_rows_equal_alone():
    """A decode row and a prompt give the same bits batched together as alone."""
    q, pre = _mixed_lengths(20, 9)
    spec = PrefillSpec("mixed-alone", 16, 8, 128, "bf16", 256, q_len_range=(1, 1),
                       q_lens=q, prefix_lens=pre)
    case = make_prefill(spec, 93)
    ref = bits(run_prefill(case)[0])
    cq = case.cu_seqlens_q
    for b in (0, 1, len(q) // 2, len(q) - 1):
        alone = run_prefill(prefill_subset(case, [b], perm_seed=b + 5))[0]
        assert np.array_equal(bits(alone), ref[cq[b]:cq[b + 1]]), b


def test_decode_rows_only():
    """A batch of decode rows only (every Lq = 1) through the varlen call."""
    rng = np.random.default_rng(10)
    n = 64
    pre = tuple(int(x) - 1 for x in rng.integers(100, 2048, n, endpoint=True))
    spec = PrefillSpec("decode-as-varlen", 16, 8, 128, "bf16", 256, q_len_range=(1, 1),
                       q_lens=(1,) * n, prefix_lens=pre)
    case = make_prefill(spec, 94)
    out, _, _ = run_prefill(case)
    assert_close(f64(out), _oracle(case), "bf16", "decode rows via varlen")
