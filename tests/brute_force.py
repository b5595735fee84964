"""Textbook attention in pure Python, on contiguous (unpaged) rows.

Used only to pin the fp64 oracle on tiny inputs: scalar loops, math.exp, no
numpy, no block tables, no slots.  It shares nothing with the oracle beyond
the definition of softmax attention.
"""
import math
import struct


def value(x, dtype):
    """Python float of one stored element (bf16 bit pattern or float32)."""
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    return float(x)


def row(vec, dtype):
    return [value(x, dtype) for x in vec]


def attend(q, keys, values, scale):
    """q: list[D]; keys/values: list of list[D] (the visible keys, in order)."""
    scores = []
    for k in keys:
        acc = 0.0
        for a, b in zip(q, k):
            acc += a * b
        scores.append(scale * acc)
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = sum(weights)
    out = []
    for d in range(len(q)):
        acc = 0.0
        for w, v in zip(weights, values):
            acc += w * v[d]
        out.append(acc / total)
    return out


def decode_seq(q_heads, keys, values, num_kv_heads, scale):
    """One sequence: q_heads [Hq][D]; keys/values [L][Hkv][D]."""
    group = len(q_heads) // num_kv_heads
    out = []
    for h, q in enumerate(q_heads):
        g = h // group
        out.append(attend(q, [k[g] for k in keys], [v[g] for v in values], scale))
    return out


def prefill_seq(q_rows, keys, values, num_kv_heads, scale):
    """One sequence: q_rows [Lq][Hq][D]; keys/values [Lk][Hkv][D] with the new
    tokens last; new row i sees keys 0 .. Lk - Lq + i."""
    lq, lk = len(q_rows), len(keys)
    out = []
    for i, q_heads in enumerate(q_rows):
        n = lk - lq + i + 1
        out.append(decode_seq(q_heads, keys[:n], values[:n], num_kv_heads, scale))
    return out
