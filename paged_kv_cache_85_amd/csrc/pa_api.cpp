// libpa C ABI: argument validation, optional host-side index checks, and
// kernel dispatch.  See include/pa.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int k = 0;
  while ((1 << k) < v) ++k;
  return k;
}

int elem_bytes(int32_t dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

bool checks_enabled() {
  const char* e = getenv("PA_CHECK");
  return e && e[0] && strcmp(e, "0") != 0;
}

// Copy n int32 values from the device (synchronising `stream`).
bool fetch(std::vector<int32_t>& dst, const int32_t* src, long long n, hipStream_t stream) {
  dst.resize((size_t)n);
  if (n == 0) return true;
  if (hipStreamSynchronize(stream) != hipSuccess) return false;
  return hipMemcpy(dst.data(), src, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost) ==
         hipSuccess;
}

bool blocks_ok(const std::vector<int32_t>& bt, int b, int mb, long long n_tokens, int bs,
               int nb) {
  const long long used = (n_tokens + bs - 1) / bs;
  for (long long i = 0; i < used; ++i) {
    const int32_t id = bt[(size_t)b * mb + i];
    if (id < 0 || id >= nb) return false;
  }
  return true;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : PA_E_HIP;
}

}  // namespace

// The attention kernels move element rows in whole 16-byte pieces.
static bool rows_aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_E_INVAL: return "invalid argument";
    case PA_E_UNSUPPORTED: return "unsupported head_dim, dtype or shape";
    case PA_E_WORKSPACE: return "workspace too small";
    case PA_E_HIP: return "HIP runtime error";
    case PA_E_NOMEM: return "not enough free blocks";
    default: return "unknown status";
  }
}

int pa_store_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || num_blocks < 1 || block_size < 1)
    return PA_E_INVAL;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_E_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_E_INVAL;
  const long long num_slots = (long long)num_blocks * block_size;
  if (num_slots > INT32_MAX) return PA_E_INVAL;  // slots are int32
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (checks_enabled()) {
    std::vector<int32_t> slots;
    if (!fetch(slots, slot_mapping, num_tokens, s)) return PA_E_HIP;
    std::vector<int32_t> seen;
    for (int32_t x : slots) {
      if (x >= num_slots) return PA_E_INVAL;
      if (x >= 0) seen.push_back(x);
    }
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return PA_E_INVAL;
  }
  const long long row_bytes = (long long)num_kv_heads * head_dim * elem_bytes(dtype);
  if (pa::launch_store_kv(k, v, k_cache, v_cache, slot_mapping, num_tokens, row_bytes,
                          num_slots, s))
    return PA_E_INVAL;
  return launch_status();
}

int pa_qk_norm_rope_store(void* q_out, const void* q, const void* k, const void* v,
                          const void* q_weight, const void* k_weight, const float* cos_sin,
                          const int32_t* positions, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                          int32_t block_size, int32_t max_position, float eps, int32_t dtype,
                          void* stream) {
  if (num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 1 ||
      block_size < 1 || max_position < 1 || !isfinite(eps) || eps < 0.f)
    return PA_E_INVAL;
  if (head_dim != 64 && head_dim != 128) return PA_E_UNSUPPORTED;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_E_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  const void* ptrs[] = {q_out, q, k, v, q_weight, k_weight, cos_sin, positions, k_cache,
                        v_cache, slot_mapping};
  for (const void* p : ptrs)
    if (!p) return PA_E_INVAL;
  // 16-byte rows of elements and of the cos/sin table are read whole.
  for (const void* p : {(const void*)q_out, q, k, v, q_weight, k_weight, (const void*)cos_sin,
                        (const void*)k_cache, (const void*)v_cache})
    if (reinterpret_cast<uintptr_t>(p) & 15) return PA_E_INVAL;
  const long long num_slots = (long long)num_blocks * block_size;
  if (num_slots > INT32_MAX) return PA_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (checks_enabled()) {
    std::vector<int32_t> slots, pos;
    if (!fetch(slots, slot_mapping, num_tokens, s)) return PA_E_HIP;
    if (!fetch(pos, positions, num_tokens, s)) return PA_E_HIP;
    std::vector<int32_t> seen;
    for (int32_t x : slots) {
      if (x >= num_slots) return PA_E_INVAL;
      if (x >= 0) seen.push_back(x);
    }
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return PA_E_INVAL;
    for (int32_t p : pos)
      if (p < 0 || p >= max_position) return PA_E_INVAL;
  }
  pa::PrologueArgs a{};
  a.q_out = q_out;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_weight = q_weight;
  a.k_weight = k_weight;
  a.cos_sin = cos_sin;
  a.positions = positions;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_position = max_position;
  a.eps = eps;
  a.num_slots = num_slots;
  if (pa::launch_store_prologue(a, head_dim, dtype == PA_DTYPE_BF16, s)) return PA_E_INVAL;
  return launch_status();
}

}  // extern "C"

// The decode workspace starts with the persistent kernel's work counter, at
// a fixed place whatever the sizes of the call, then the split-context
// partials of kDecodePartition-token partitions:
// [work counter: 256 B][partial outputs][partial max / sum].
constexpr size_t kCounterBytes = 256;

struct DecodeLayout {
  int max_parts;   // partitions of the longest context
  size_t ml_off;   // byte offset of the (max, sum) pairs
  size_t total;    // bytes
};

static DecodeLayout decode_layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len) {
  DecodeLayout l{};
  l.max_parts = (int)(((long long)max_context_len + pa::kDecodePartition - 1) /
                      pa::kDecodePartition);
  const size_t heads = (size_t)num_seqs * num_q_heads;
  const size_t o_bytes = heads * (size_t)l.max_parts * head_dim * sizeof(float);
  l.ml_off = (kCounterBytes + o_bytes + 255) & ~(size_t)255;
  l.total = l.ml_off + heads * (size_t)l.max_parts * 2 * sizeof(float);
  return l;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  return decode_layout(num_seqs, num_q_heads, head_dim, max_context_len).total;
}

static int heads_per_wg(int group, int head_dim) {
  const int cap = head_dim == 64 ? 8 : 4;
  for (int hg = std::min(group, cap); hg > 1; --hg)
    if (group % hg == 0) return hg;
  return 1;
}

// Work counters must be zero when a call starts (each call leaves them so).
// Under PA_CHECK the first `n` 32-byte-spaced counters are read back.
static int counters_zero(const void* workspace, int n, hipStream_t s) {
  std::vector<int32_t> c;
  if (!fetch(c, static_cast<const int32_t*>(workspace), (long long)n * 8, s)) return PA_E_HIP;
  for (int i = 0; i < n; ++i)
    if (c[(size_t)i * 8] != 0) return PA_E_WORKSPACE;
  return PA_OK;
}

namespace pa {

int decode_entry(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                 int32_t max_context_len, float scale, int32_t dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t s) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 1 ||
      block_size < 1 || max_blocks_per_seq < 1 || max_context_len < 1 || !isfinite(scale) ||
      !(scale > 0.f))
    return PA_E_INVAL;
  if (num_q_heads % num_kv_heads) return PA_E_INVAL;
  if (head_dim != 64 && head_dim != 128) return PA_E_UNSUPPORTED;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_E_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size < max_context_len) return PA_E_INVAL;
  if ((long long)num_blocks * block_size > INT32_MAX) return PA_E_INVAL;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_E_INVAL;
  if (!rows_aligned16({out, q, k_cache, v_cache})) return PA_E_INVAL;

  const int group = num_q_heads / num_kv_heads;
  const int hg = heads_per_wg(group, head_dim);
  const DecodeLayout lay = decode_layout(num_seqs, num_q_heads, head_dim, max_context_len);
  if (lay.max_parts > 1) {
    if (!workspace || workspace_bytes < lay.total) return PA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PA_E_INVAL;
  }
  if (checks_enabled()) {
    std::vector<int32_t> lens, bt;
    if (!fetch(lens, context_lens, num_seqs, s)) return PA_E_HIP;
    if (!fetch(bt, block_tables, (long long)num_seqs * max_blocks_per_seq, s)) return PA_E_HIP;
    for (int b = 0; b < num_seqs; ++b) {
      if (lens[b] < 1 || lens[b] > max_context_len) return PA_E_INVAL;
      if (!blocks_ok(bt, b, max_blocks_per_seq, lens[b], block_size, num_blocks))
        return PA_E_INVAL;
    }
    if (lay.max_parts > 1) {
      const int rc = counters_zero(workspace, 1, s);
      if (rc != PA_OK) return rc;
    }
  }

  pa::RowAttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  if (lay.max_parts > 1) {
    a.ticket = static_cast<unsigned*>(workspace);
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml_off);
  }
  a.num_rows = num_seqs;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.heads_per_wg = hg;
  a.head_chunks = group / hg;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.block_size_log2 = log2_exact(block_size);
  a.max_context = max_context_len;
  a.part_tokens = pa::kDecodePartition;
  a.max_parts = lay.max_parts;
  a.scale_log2 = (float)((double)scale * kLog2e);
  if (pa::launch_decode(a, head_dim, dtype, s)) return PA_E_UNSUPPORTED;
  return launch_status();
}

size_t decode_scratch_need(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                           int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const DecodeLayout l = decode_layout(num_seqs, num_q_heads, head_dim, max_context_len);
  return l.max_parts > 1 ? l.total : 0;
}

}  // namespace pa

extern "C" {

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
              int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
              float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
              void* stream) {
  return pa::decode_entry(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq, max_context_len, scale, dtype, workspace,
                          workspace_bytes, static_cast<hipStream_t>(stream));
}

int pa_prefill_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float scale,
                      int32_t dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
      num_q_heads < 1 || num_kv_heads < 1 || num_blocks < 1 || block_size < 1 ||
      max_blocks_per_seq < 1 || !isfinite(scale) || !(scale > 0.f))
    return PA_E_INVAL;
  if (num_q_heads % num_kv_heads) return PA_E_INVAL;
  if (head_dim != 64 && head_dim != 128) return PA_E_UNSUPPORTED;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_E_UNSUPPORTED;
  if (max_seqlen_q > max_seqlen_k) return PA_E_INVAL;
  if ((long long)max_blocks_per_seq * block_size < max_seqlen_k) return PA_E_INVAL;
  if ((long long)num_blocks * block_size > INT32_MAX) return PA_E_INVAL;
  if (workspace) {
    if (workspace_bytes < PA_PREFILL_WORKSPACE_BYTES) return PA_E_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PA_E_INVAL;
  }
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !cu_seqlens_k)
    return PA_E_INVAL;
  if (!rows_aligned16({out, q, k_cache, v_cache})) return PA_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (checks_enabled()) {
    std::vector<int32_t> cq, ck, bt;
    if (!fetch(cq, cu_seqlens_q, num_seqs + 1, s)) return PA_E_HIP;
    if (!fetch(ck, cu_seqlens_k, num_seqs + 1, s)) return PA_E_HIP;
    if (!fetch(bt, block_tables, (long long)num_seqs * max_blocks_per_seq, s)) return PA_E_HIP;
    if (cq[0] != 0 || ck[0] != 0 || cq[num_seqs] != total_q) return PA_E_INVAL;
    for (int b = 0; b < num_seqs; ++b) {
      const int lq = cq[b + 1] - cq[b], lk = ck[b + 1] - ck[b];
      if (lq < 0 || lk < lq || lq > max_seqlen_q || lk > max_seqlen_k) return PA_E_INVAL;
      if (!blocks_ok(bt, b, max_blocks_per_seq, lk, block_size, num_blocks)) return PA_E_INVAL;
    }
    if (workspace && dtype == PA_DTYPE_BF16) {
      const int rc = counters_zero(workspace, 8, s);
      if (rc != PA_OK) return rc;
    }
  }
  const int group = num_q_heads / num_kv_heads;
  if (dtype == PA_DTYPE_BF16) {
    pa::PrefillArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.cu_seqlens_q = cu_seqlens_q;
    a.cu_seqlens_k = cu_seqlens_k;
    a.out = out;
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.block_size_log2 = log2_exact(block_size);
    a.scale_log2 = (float)((double)scale * kLog2e);
    a.ticket = static_cast<unsigned*>(workspace);
    if (pa::launch_prefill_bf16(a, head_dim, s)) return PA_E_UNSUPPORTED;
    return launch_status();
  }
  // fp32: every packed row is a decode over its causal context, one
  // partition per row (no workspace).
  pa::RowAttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.out = out;
  a.num_rows = total_q;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.heads_per_wg = heads_per_wg(group, head_dim);
  a.head_chunks = group / a.heads_per_wg;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.block_size_log2 = log2_exact(block_size);
  a.max_context = max_seqlen_k;
  a.part_tokens = std::max(64, ((max_seqlen_k + 63) / 64) * 64);
  a.max_parts = 1;
  a.scale_log2 = (float)((double)scale * kLog2e);
  if (pa::launch_varlen_rows(a, head_dim, dtype, s)) return PA_E_UNSUPPORTED;
  return launch_status();
}

}  // extern "C"
