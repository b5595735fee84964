"""fp64 CPU oracle for paged-KV attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP path.
"""
from .paged_attention import decode, gather, prefill_varlen, store_kv, widen
from .store_prologue import qk_norm_rope, qk_norm_rope_store, rms_norm, rope

__all__ = ["decode", "gather", "prefill_varlen", "qk_norm_rope", "qk_norm_rope_store",
           "rms_norm", "rope", "store_kv", "widen"]
