"""Seeded synthetic workloads for paged-KV attention (inputs only, no attention arithmetic)."""
from .generate import (CONFIGS, DecodeCase, DecodeSpec, PrefillCase, PrefillSpec, PrologueCase,
                       bf16_bits, decode_subset, logical_prefix, make_case, make_decode,
                       make_prefill, make_prologue, prefill_subset, poison_bits, rope_table,
                       storage_np_dtype, token_rows)

__all__ = ["CONFIGS", "DecodeCase", "DecodeSpec", "PrefillCase", "PrefillSpec", "bf16_bits",
           "decode_subset", "logical_prefix", "make_case", "make_decode", "make_prefill",
           "poison_bits", "prefill_subset", "storage_np_dtype", "PrologueCase", "make_prologue",
           "rope_table", "token_rows"]
