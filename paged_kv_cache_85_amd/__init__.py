"""Attention over a paged KV cache on MI355X (gfx950): Python face of libpa.

The three calls of the hot path -- pa_store_kv, pa_decode and
pa_prefill_varlen -- run in hand-written HIP kernels behind the C ABI in
include/pa.h; this package only marshals torch device tensors into that ABI.
"""
from .binding import (EXPORTS, LIB_PATH, PA_DTYPE_BF16, PA_DTYPE_F32, PA_E_HIP, PA_E_INVAL,
                      PA_E_NOMEM, PA_E_UNSUPPORTED, PA_E_WORKSPACE, PA_OK, BlockManager, PAError,
                      lib, pa_decode, pa_decode_noalloc,
                      pa_decode_workspace_bytes, pa_prefill_varlen, pa_qk_norm_rope_store,
                      pa_status_string, pa_store_kv)

__all__ = ["BlockManager", "PA_E_NOMEM",
           "EXPORTS", "LIB_PATH", "PA_DTYPE_BF16", "PA_DTYPE_F32", "PA_E_HIP", "PA_E_INVAL",
           "PA_E_UNSUPPORTED", "PA_E_WORKSPACE", "PA_OK", "PAError", "lib", "pa_decode",
           "pa_decode_noalloc",
           "pa_decode_workspace_bytes", "pa_prefill_varlen", "pa_qk_norm_rope_store",
           "pa_status_string", "pa_store_kv"]
