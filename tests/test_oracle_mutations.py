"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only).

Each mutation is a textual edit of the oracle's source; the edited copy is
executed as a throw-away module and run through the pin checks.  A mutation
survives only if every check passes on it, which would mean the pins do not
constrain that part of the oracle.
"""
import os
import types

import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "paged_attention.py")

# (id, text to find, replacement, which occurrence (None = the only one))
MUTATIONS = [
    ("decode-gqa-modulo", "g = h // group", "g = h % num_kv_heads", 0),
    ("prefill-gqa-modulo", "g = h // group", "g = h % num_kv_heads", 1),
    ("decode-drops-scale", "scores = scale * (keys[:, g, :] @ q_vec)",
     "scores = (keys[:, g, :] @ q_vec)", None),
    ("prefill-drops-scale", "S = scale * (qh @ keys[:, g, :].T)", "S = (qh @ keys[:, g, :].T)",
     None),
    ("causal-top-left", "visible = cols <= (lk - lq) + rows", "visible = cols <= rows", None),
    ("causal-off-by-one", "visible = cols <= (lk - lq) + rows",
     "visible = cols < (lk - lq) + rows", None),
    ("causal-unmasked", "S = np.where(visible, S, -np.inf)", "S = S", None),
    ("gather-ignores-table", "return pool[table_row[pos // bs], pos % bs]",
     "return pool[pos // bs, pos % bs]", None),
    ("gather-swapped-index", "return pool[table_row[pos // bs], pos % bs]",
     "return pool[table_row[pos % bs], pos // bs]", None),
    ("softmax-sign", "p = np.exp(scores - m)", "p = np.exp(m - scores)", None),
    ("decode-reads-keys-as-values", "out[b, h] = (p @ values[:, g, :]) / p.sum()",
     "out[b, h] = (p @ keys[:, g, :]) / p.sum()", None),
    ("decode-unnormalised", "out[b, h] = (p @ values[:, g, :]) / p.sum()",
     "out[b, h] = (p @ values[:, g, :])", None),
    ("prefill-max-wrong-axis", "m = S.max(axis=1, keepdims=True)",
     "m = S.max(axis=0, keepdims=True)", None),
    ("prefill-global-sum", "/ P.sum(axis=1, keepdims=True)", "/ P.sum()", None),
    ("prefill-reads-keys-as-values", "(P @ values[:, g, :])", "(P @ keys[:, g, :])", None),
    ("decode-drops-new-token", "L = int(context_lens[b])", "L = int(context_lens[b]) - 1", None),
    ("prefill-wrong-query-head", "qh = widen(q[q0:q1, h, :], dtype)",
     "qh = widen(q[q0:q1, g, :], dtype)", None),
    ("store-swapped-index", "kc[s // bs, s % bs] = k[t]", "kc[s % bs, s // bs] = k[t]", None),
    ("store-v-gets-k", "vc[s // bs, s % bs] = v[t]", "vc[s // bs, s % bs] = k[t]", None),
    ("store-drops-slot-zero", "if s < 0:", "if s <= 0:", None),
    ("store-writes-padding", "if s < 0:\n            continue", "if False:\n            continue",
     None),
    ("bf16-widen-shift", "<< 16", "<< 15", None),
    ("prefill-key-length-from-q", "lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])",
     "lk = int(cu_seqlens_q[b + 1]) - int(cu_seqlens_q[b])", None),
]


def _mutant(find, repl, occurrence):
    with open(ORACLE_SRC) as f:
        src = f.read()
    n = src.count(find)
    if occurrence is None:
        assert n == 1, f"pattern must occur once, found {n}: {find!r}"
        src = src.replace(find, repl)
    else:
        assert n > occurrence, f"pattern occurs {n} times: {find!r}"
        at = -1
        for _ in range(occurrence + 1):
            at = src.index(find, at + 1)
        src = src[:at] + repl + src[at + len(find):]
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "<oracle mutant>", "exec"), mod.__dict__)
    return mod


# A planted mistake may turn a masked score into NaN (the off-by-one mask
# leaves a row with no visible key); that is the mutant's behaviour, not a
# warning about the oracle.
@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("mid,find,repl,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(mid, find, repl, occ):
    mod = _mutant(find, repl, occ)
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:          # an assertion or a crash: the mistake is caught
            return
    pytest.fail(f"mutation {mid!r} passed every pin")


# ---- the store-prologue oracle (QK RMS norm, rotary embedding, K/V store)
import rope_pins

PROLOGUE_SRC = os.path.join(os.path.dirname(ORACLE_SRC), "store_prologue.py")
PROLOGUE_MUTATIONS = [
    ("rms-drops-eps", "np.sqrt(ms + eps)", "np.sqrt(ms)"),
    ("rms-wrong-axis", "np.mean(x * x, axis=-1, keepdims=True)", "np.mean(x * x, axis=-2, keepdims=True)"),
    ("rms-drops-gain", "/ np.sqrt(ms + eps) * w", "/ np.sqrt(ms + eps)"),
    ("rope-sin-sign", "out[t, :, :half] = a * c - b * s", "out[t, :, :half] = a * c + b * s"),
    ("rope-second-half-sign", "out[t, :, half:] = b * c + a * s", "out[t, :, half:] = b * c - a * s"),
    ("rope-sin-cos-swapped", "c = cos_sin[positions[t], :half]", "c = cos_sin[positions[t], half:]"),
    ("rope-position-off-by-one", "c = cos_sin[positions[t], :half]\n        s = cos_sin[positions[t], half:]",
     "c = cos_sin[positions[t] + 1, :half]\n        s = cos_sin[positions[t] + 1, half:]"),
    ("rope-interleaved-pairs", "a, b = y[t, :, :half], y[t, :, half:]", "a, b = y[t, :, 0::2], y[t, :, 1::2]"),
    ("store-v-skips-slot-zero", "if s >= 0:", "if s > 0:"),
    ("key-uses-query-gain", "rms_norm(kf, wk, eps)", "rms_norm(kf, wq, eps)"),
]


@pytest.mark.parametrize("mid,find,repl", PROLOGUE_MUTATIONS, ids=[m[0] for m in PROLOGUE_MUTATIONS])
def test_prologue_mutation_is_caught(mid, find, repl):
    with open(PROLOGUE_SRC) as f:
        src = f.read()
    assert src.count(find) == 1, find
    src = src.replace(find, repl).replace("from .paged_attention import widen",
                                          "from oracle.paged_attention import widen")
    mod = types.ModuleType("prologue_mutant")
    exec(compile(src, "<prologue mutant>", "exec"), mod.__dict__)
    for check in rope_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:
            return
    pytest.fail(f"mutation {mid!r} passed every pin")


# ---- the block-manager model (free list, prefix cache, slots)
import test_block_manager

BM_SRC = os.path.join(os.path.dirname(ORACLE_SRC), "block_manager.py")
BM_MUTATIONS = [
    ("full-hit-not-recomputed", "cached = min(cached, n - 1)", "cached = cached"),
    ("free-list-lifo", "self.free.popitem(last=False)", "self.free.popitem(last=True)"),
    ("reused-block-keeps-key", "del self.registry[self.key[b]]", "pass"),
    ("release-front-to-back", 'for b in reversed(s["blocks"]):', 'for b in s["blocks"]:'),
    ("slot-offset", "return b * bs + n % bs", "return b * bs + (n + 1) % bs"),
    ("append-never-registers", 'self._register(b, tuple(s["tokens"][:n + 1]))', "pass"),
    ("partial-block-cached", ("for i in range(n // bs):", "if (i + 1) * bs <= n:"),
     ("for i in range(nblocks):", "if True:")),
    ("hit-stays-on-free-list", "del self.free[b]\n", "pass\n"),
    ("release-ignores-refcount", "if self.ref[b] == 0:", "if True:"),
]


@pytest.mark.parametrize("mid,find,repl", BM_MUTATIONS, ids=[m[0] for m in BM_MUTATIONS])
def test_block_model_mutation_is_caught(mid, find, repl):
    with open(BM_SRC) as f:
        src = f.read()
    finds, repls = (find, repl) if isinstance(find, tuple) else ((find,), (repl,))
    for f_, r_ in zip(finds, repls):
        assert src.count(f_) == 1, f_
        src = src.replace(f_, r_)
    # the mutant raises the real shortage error, so the checks recognise it
    src = src.replace("class NoMemory(Exception):\n    pass", "from oracle.block_manager import NoMemory")
    mod = types.ModuleType("block_mutant")
    exec(compile(src, "<block-manager mutant>", "exec"), mod.__dict__)
    for check in test_block_manager.MODEL_PINS + [test_block_manager.model_invariants]:
        try:
            check(mod.BlockModel)
        except (Exception, pytest.fail.Exception):  # a missing pytest.raises error is a catch
            return
    pytest.fail(f"mutation {mid!r} passed every pin")
