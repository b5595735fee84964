"""fp64 CPU oracle for the store prologue: query/key RMS normalisation and
rotary position embedding, then the K/V store.

TEST INFRASTRUCTURE ONLY (same rule as the attention oracle): only the tests,
the package smoke check and the benchmark's CPU-baseline leg may use it, and
it shares no code with the HIP path.

What it computes, and where the pages say so:

* QK normalisation -- Qwen3 normalises queries and keys per head before
  attention (the smzdm Nano-vLLM walk-through, model implementation details).
  The pages give no formula; the plain reading is an RMS norm over each
  head's head_dim elements with a learned per-element gain:
      y_i = x_i / sqrt(mean_j(x_j^2) + eps) * w_i.
* Rotary embedding -- the model rotates queries and keys by their position
  ("mini-vLLM", project summary: rotary embeddings).  No variant is named;
  the plain reading is the half-split ("neox") rotation with a cos/sin table
  indexed by position: for i < D/2, with c = cos[p][i], s = sin[p][i],
      out_i       = y_i * c - y_{i+D/2} * s
      out_{i+D/2} = y_{i+D/2} * c + y_i * s.
  The table is an input ([max_position, D] float32: cos in the first D/2
  columns, sin in the last D/2), so both sides rotate by the same numbers.
* Store -- the normalised, rotated key row and the raw value row go to the
  slot the slot mapping names; negative slots are skipped (as store_kv).

Everything is evaluated in float64 on the exact input values; the result is
the unrounded float64 value (the GPU rounds once, to the storage dtype).

Pins (CPU suite): unit gain gives rows of RMS sqrt(ms / (ms + eps)); position
0 is the identity; rotation keeps each (i, i + D/2) pair's length; the
dot product of a rotated query and key depends only on the distance between
their positions (the defining property of rotary embeddings) for a table
built from the usual frequencies; a hand-worked D = 4 example.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import widen

__all__ = ["rms_norm", "rope", "qk_norm_rope", "qk_norm_rope_store"]


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x: [..., D] float64, w: [D] float64 -> x / sqrt(mean(x^2) + eps) * w."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope(y: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """y: [T, H, D] float64; positions: [T]; cos_sin: [P, D] float64 -> rotated [T, H, D]."""
    T, H, D = y.shape
    half = D // 2
    out = np.empty_like(y)
    for t in range(T):
        c = cos_sin[positions[t], :half]
        s = cos_sin[positions[t], half:]
        a, b = y[t, :, :half], y[t, :, half:]
        out[t, :, :half] = a * c - b * s
        out[t, :, half:] = b * c + a * s
    return out


def qk_norm_rope(q, k, q_weight, k_weight, positions, cos_sin, eps, dtype):
    """Normalised, rotated queries and keys (float64), from stored inputs."""
    qf, kf = widen(q, dtype), widen(k, dtype)
    wq, wk = widen(q_weight, dtype), widen(k_weight, dtype)
    cs = np.asarray(cos_sin, np.float32).astype(np.float64)
    pos = np.asarray(positions, np.int64)
    return (rope(rms_norm(qf, wq, eps), pos, cs), rope(rms_norm(kf, wk, eps), pos, cs))


def qk_norm_rope_store(q, k, v, q_weight, k_weight, positions, cos_sin, eps, v_cache,
                       slot_mapping, dtype):
    """Returns (q_out float64 [T, Hq, D], key rows float64 [T, Hkv, D], new
    v_cache): the key rows are what each non-negative slot must hold after
    rounding; the value pool is updated byte for byte."""
    q_out, k_out = qk_norm_rope(q, k, q_weight, k_weight, positions, cos_sin, eps, dtype)
    vc = np.array(v_cache, copy=True)
    bs = vc.shape[1]
    for t, s in enumerate(np.asarray(slot_mapping)):
        if s >= 0:
            vc[s // bs, s % bs] = v[t]
    return q_out, k_out, vc
