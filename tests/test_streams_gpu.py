"""Calls on a stream other than torch's current one, with the binding's own
default workspaces: the workspace is made and zeroed on the stream the kernel
runs on, so the result is the current-stream result, bit for bit, and the
work counters come back to zero."""
import numpy as np
import pytest
import torch

import paged_kv_cache_85_amd as pa
from paged_kv_cache_85_amd import binding
from gpu_harness import bits, dev, say
from synth import make_case

pytestmark = pytest.mark.gpu


def test_decode_and_prefill_on_a_side_stream():
    side = torch.cuda.Stream()
    c = make_case(3)
    kc, vc = dev(c.k_cache), dev(c.v_cache)
    pa.pa_store_kv(dev(c.k_new), dev(c.v_new), kc, vc, dev(c.slot_mapping))
    q, bt, cl = dev(c.q), dev(c.block_tables), dev(c.context_lens)
    ref = torch.empty_like(q)
    pa.pa_decode(ref, q, kc, vc, bt, cl, c.max_context_len, float(c.scale))
    say("decode on a side stream, binding workspace")
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        o = torch.empty_like(q)
        pa.pa_decode(o, q, kc, vc, bt, cl, c.max_context_len, float(c.scale), stream=side)
        outs.append(o)
    side.synchronize()
    for o in outs:
        assert np.array_equal(bits(o), bits(ref))
    key = (0, side.cuda_stream)
    assert int(binding._decode_ws[key][:256].count_nonzero()) == 0

    p = make_case(4)
    kc, vc = dev(p.k_cache), dev(p.v_cache)
    pa.pa_store_kv(dev(p.k_new), dev(p.v_new), kc, vc, dev(p.slot_mapping))
    q, bt, cq, ck = dev(p.q), dev(p.block_tables), dev(p.cu_seqlens_q), dev(p.cu_seqlens_k)
    ref = torch.empty_like(q)
    pa.pa_prefill_varlen(ref, q, kc, vc, bt, cq, ck, p.max_seqlen_q, p.max_seqlen_k,
                         float(p.scale))
    say("prefill on a side stream, binding work counters")
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(2):
        o = torch.empty_like(q)
        pa.pa_prefill_varlen(o, q, kc, vc, bt, cq, ck, p.max_seqlen_q, p.max_seqlen_k,
                             float(p.scale), stream=side)
        outs.append(o)
    side.synchronize()
    for o in outs:
        assert np.array_equal(bits(o), bits(ref))
    assert int(binding._prefill_ws[key].count_nonzero()) == 0
