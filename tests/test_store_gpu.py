"""pa_store_kv on the GPU: bit-exact against the oracle's store on every
workload, negative slots skipped, every other pool byte unchanged."""
import numpy as np
import pytest

import oracle
from gpu_harness import bits, run_store, say
from synth import DecodeSpec, make_case, make_decode

pytestmark = pytest.mark.gpu


def _expect(case, slots=None):
    sm = case.slot_mapping if slots is None else np.asarray(slots, np.int32)
    return oracle.store_kv(case.k_cache, case.v_cache, case.k_new, case.v_new, sm)


def _raw(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_store_bit_exact(config):
    case = make_case(config)
    say(f"store config {config}: T={len(case.slot_mapping)} NB={case.num_blocks} "
        f"BS={case.block_size}")
    kc, vc = run_store(case)
    ek, ev = _expect(case)
    assert np.array_equal(bits(kc), _raw(ek))
    assert np.array_equal(bits(vc), _raw(ev))


@pytest.mark.parametrize("dtype,head_dim,heads", [("f32", 64, 1), ("bf16", 64, 2), ("f32", 3, 5),
                                                  ("bf16", 5, 3), ("bf16", 128, 8)])
def test_store_padding_and_odd_rows(dtype, head_dim, heads):
    spec = DecodeSpec("store-odd", heads, heads, head_dim, dtype, 4,
                      context_lens=(1, 5, 8, 9, 3, 12))
    case = make_decode(spec, 61)
    slots = case.slot_mapping.copy()
    slots[1] = -1                         # padding rows are skipped
    slots[4] = -7
    say(f"store odd rows {dtype} D={head_dim} Hkv={heads}")
    kc, vc = run_store(case, slots)
    ek, ev = _expect(case, slots)
    assert np.array_equal(bits(kc), _raw(ek))
    assert np.array_equal(bits(vc), _raw(ev))


def test_store_skips_out_of_range_slot():
    spec = DecodeSpec("store-oob", 2, 2, 64, "bf16", 4, context_lens=(2, 3))
    case = make_decode(spec, 62)
    slots = case.slot_mapping.copy()
    slots[1] = case.num_blocks * case.block_size   # one past the pool: documented as skipped
    kc, vc = run_store(case, slots)
    slots[1] = -1
    ek, ev = _expect(case, slots)
    assert np.array_equal(bits(kc), _raw(ek))
    assert np.array_equal(bits(vc), _raw(ev))
