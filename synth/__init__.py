"""Seeded synthetic workloads for paged-KV attention (inputs only, no attention arithmetic)."""
from .generate import (CONFIGS, DecodeCase, DecodeSpec, PrefillCase, PrefillSpec, bf16_bits,
                       decode_subset, logical_prefix, make_case, make_decode, make_prefill, prefill_subset,
                       poison_bits, storage_np_dtype)

__all__ = ["CONFIGS", "DecodeCase", "DecodeSpec", "PrefillCase", "PrefillSpec", "bf16_bits",
           "decode_subset", "logical_prefix", "make_case", "make_decode", "make_prefill",
           "poison_bits", "prefill_subset", "storage_np_dtype"]
