"""Pins of the store-prologue oracle (RMS norm of queries and keys per head,
half-split rotary embedding, K/V store), written as checks that take an oracle
module, so that the mutation suite can run them on edited copies.  Each check
rests on a property or a worked example, not on the oracle's own code."""
import json
import os

import numpy as np

from synth import make_prologue, rope_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qk_norm_rope_d4.json")


def check_worked_example_d4(m):
    g = json.load(open(GOLDEN))
    x = np.array(g["x"], np.float64)[None, None, :]
    w = np.array(g["weight"], np.float64)
    y = m.rms_norm(x, w, g["eps"])
    table = np.array([[1.0, 1.0, 0.0, 0.0], g["cos"] + g["sin"]], np.float64)
    out = m.rope(y, np.array([1]), table)
    assert np.allclose(out[0, 0], g["expected"], atol=1e-12)
    # position 0 of the same table is the identity
    assert np.allclose(m.rope(y, np.array([0]), table), y, atol=0)


def check_unit_gain_rms(m):
    """With unit gain every head row has mean square ms / (ms + eps), where ms
    is that row's own mean square (so normalising over the wrong axis fails)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 64)) * rng.uniform(0.1, 10, (5, 3, 1))
    eps = 1e-3
    y = m.rms_norm(x, np.ones(64), eps)
    ms = (x ** 2).sum(-1) / 64
    assert np.allclose((y ** 2).sum(-1) / 64, ms / (ms + eps), rtol=1e-12)
    # and a gain scales each element
    wv = rng.uniform(0.5, 2, 64)
    assert np.allclose(m.rms_norm(x, wv, eps), y * wv, rtol=1e-12)


def check_rotation_keeps_pair_lengths_and_identity_at_zero(m):
    rng = np.random.default_rng(2)
    D = 128
    y = rng.standard_normal((7, 4, D))
    table = rope_table(4096, D).astype(np.float64)
    pos = rng.integers(0, 4096, 7)
    r = m.rope(y, pos, table)
    h = D // 2
    assert np.allclose(r[..., :h] ** 2 + r[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2,
                       rtol=1e-6)   # the float32 table's cos^2 + sin^2 is 1 to ~1e-7
    assert np.allclose(m.rope(y, np.zeros(7, int), table), y, atol=0)


def check_rotary_dot_depends_on_distance_only(m):
    """<R(m) q, R(n) k> = <R(m + s) q, R(n + s) k>: the defining property,
    which holds only if both halves rotate by the same per-frequency angle."""
    rng = np.random.default_rng(3)
    D = 64
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    table = rope_table(3000, D, theta=10000.0).astype(np.float64)
    base = None
    for shift in (0, 17, 500, 2000):
        pm, pn = 40 + shift, 13 + shift
        d = float((m.rope(q, np.array([pm]), table) * m.rope(k, np.array([pn]), table)).sum())
        base = d if base is None else base
        assert abs(d - base) < 1e-5 * max(1.0, abs(base))


def check_table_matches_closed_form(m):
    D = 8
    t = rope_table(10, D, theta=100.0).astype(np.float64)
    for p in (0, 3, 9):
        for i in range(D // 2):
            ang = p / 100.0 ** (2 * i / D)
            assert abs(t[p, i] - np.cos(ang)) < 1e-7 and abs(t[p, D // 2 + i] - np.sin(ang)) < 1e-7


def check_store_prologue(m, config=1):
    """Values go to their slots byte for byte; negative slots are skipped;
    the outputs have the input shapes."""
    c = make_prologue(config, 12)
    slots = c.slot_mapping.copy()
    slots[0] = -1
    q_out, k_rows, vc = m.qk_norm_rope_store(c.q, c.k, c.v, c.q_weight, c.k_weight, c.positions,
                                           c.cos_sin, c.eps, c.v_cache, slots, c.dtype)
    assert q_out.shape == c.q.shape and k_rows.shape == c.k.shape
    bs = vc.shape[1]
    for t, s in enumerate(slots):
        if s >= 0:
            assert vc[s // bs, s % bs].tobytes() == c.v[t].tobytes()
    s0 = c.slot_mapping[0]   # skipped: the pool's bytes there (poison) are unchanged
    assert vc[s0 // bs, s0 % bs].tobytes() == c.v_cache[s0 // bs, s0 % bs].tobytes()
    # each output row of q is rms_norm then rope of its own row
    qf = m.widen(c.q, c.dtype)
    one = m.rope(m.rms_norm(qf[:1], m.widen(c.q_weight, c.dtype), c.eps), c.positions[:1],
               c.cos_sin.astype(np.float64))
    assert np.allclose(q_out[:1], one, atol=0)


def check_key_rows_use_key_gain(m):
    """Key rows are the key's own norm (with the key gain) then rotation."""
    c = make_prologue(1, 13)
    _, k_rows, _ = m.qk_norm_rope_store(c.q, c.k, c.v, c.q_weight, c.k_weight, c.positions,
                                        c.cos_sin, c.eps, c.v_cache, c.slot_mapping, c.dtype)
    kf = m.widen(c.k, c.dtype)
    exp = m.rope(m.rms_norm(kf, m.widen(c.k_weight, c.dtype), c.eps), c.positions,
                 c.cos_sin.astype(np.float64))
    assert np.allclose(k_rows, exp, atol=0)
    assert not np.allclose(c.q_weight, c.k_weight)


def check_value_store_slot_zero(m):
    """Slot 0 is a real slot; -1 is skipped (a 2-block pool of 2-token blocks)."""
    f = np.float32
    q = np.ones((3, 1, 4), f); k = np.ones((3, 1, 4), f)
    v = np.arange(12, dtype=f).reshape(3, 1, 4) + 1
    vc0 = np.zeros((2, 2, 1, 4), f)
    table = np.array([[1, 1, 0, 0]], f)
    _, _, vc = m.qk_norm_rope_store(q, k, v, np.ones(4, f), np.ones(4, f), np.zeros(3, np.int32),
                                    table, 0.0, vc0, np.array([0, -1, 3], np.int32), "f32")
    assert np.array_equal(vc[0, 0], v[0]) and np.array_equal(vc[1, 1], v[2])
    assert np.array_equal(vc[0, 1], vc0[0, 1]) and np.array_equal(vc[1, 0], vc0[1, 0])


def check_store_prologue_f32(m):
    check_store_prologue(m, 1)


def check_store_prologue_bf16(m):
    check_store_prologue(m, 2)


ALL_CHECKS = [check_worked_example_d4, check_unit_gain_rms,
              check_rotation_keeps_pair_lengths_and_identity_at_zero,
              check_rotary_dot_depends_on_distance_only, check_table_matches_closed_form,
              check_store_prologue_f32, check_store_prologue_bf16, check_key_rows_use_key_gain,
              check_value_store_slot_zero]
