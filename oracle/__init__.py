"""fp64 CPU oracle for paged-KV attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP path.
"""
from .paged_attention import decode, gather, prefill_varlen, store_kv, widen

__all__ = ["decode", "gather", "prefill_varlen", "store_kv", "widen"]
