// Host-side launchers of libpa's kernels (internal; the public ABI is pa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// Tokens per decode context partition.  It is fixed, not tuned to the
// batch, so a row's arithmetic depends only on its own tokens: the output is
// bitwise the same whether a sequence runs alone or batched, whatever its
// physical block IDs or the block size.  512 measured best on the Qwen3
// decode workload (256 sequences of 100..2048 tokens: 201 us against 207 us
// at 256 and 236 us at 128): fewer items per wave, half the split-context
// traffic.  Small batches, whose time is one wave's partition, pay for it
// (32 Qwen2.5 sequences: 41 us against 27 us at 256).
#ifndef PA_DECODE_PARTITION
#define PA_DECODE_PARTITION PA_DECODE_PARTITION_TOKENS
#endif
constexpr int kDecodePartition = PA_DECODE_PARTITION;

// pa_decode after its stream argument is converted (shared by the entry
// points that differ only in where the workspace comes from).
int decode_entry(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                 int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                 int32_t max_context_len, float scale, int32_t dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

// Workspace bytes decode_entry needs for these sizes (0: none).
size_t decode_scratch_need(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                           int32_t max_context_len);

int launch_store_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                    const int32_t* slot_mapping, int num_tokens, long long row_bytes,
                    long long num_slots, hipStream_t stream);

// Row-wise attention on the vector ALUs: every query row attends over its own
// context.  Decode rows come from context_lens; varlen rows (fp32 prefill)
// derive their context from cu_seqlens.
struct RowAttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;   // decode mode
  const int32_t* cu_seqlens_q;   // varlen mode
  const int32_t* cu_seqlens_k;   // varlen mode
  void* out;
  float* ws_o;                   // [rows, Hq, max_parts, D] unnormalised partial outputs
  float* ws_ml;                  // [rows, Hq, max_parts, 2] (running max in log2 units, sum)
  unsigned* ticket;              // decode work counter in the workspace (null: static deal)
  int num_rows;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                     // Hq / Hkv
  int heads_per_wg;              // query heads of one group handled together
  int head_chunks;               // group / heads_per_wg
  int max_blocks_per_seq;
  int num_blocks;
  int block_size;
  int block_size_log2;           // -1 when block_size is not a power of two
  int max_context;               // clamp for per-row context lengths
  int part_tokens;               // tokens per partition (multiple of 64)
  int max_parts;
  float scale_log2;              // scale * log2(e)
};

int launch_decode(const RowAttnArgs& a, int head_dim, int dtype, hipStream_t stream);
// Query groups from this size up take the matrix-core decode kernel (bf16).
#ifndef PA_GQA_MIN_GROUP
#define PA_GQA_MIN_GROUP 4
#endif
constexpr int kGqaMfmaMinGroup = PA_GQA_MIN_GROUP;
int gqa_mfma_heads(int group, int head_dim);
int launch_decode_gqa_mfma(const RowAttnArgs& a, int head_dim, hipStream_t stream);
int launch_varlen_rows(const RowAttnArgs& a, int head_dim, int dtype, hipStream_t stream);

struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  void* out;
  int num_seqs;
  int total_q;
  int max_seqlen_q;
  int max_seqlen_k;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int max_blocks_per_seq;
  int num_blocks;
  int block_size;
  int block_size_log2;
  float scale_log2;
  int persistent;   // set by the launcher: workgroups loop over work items
  unsigned* ticket; // work counter (null: every item dealt in a fixed order)
  int xcd_groups;   // set by the launcher: deal each KV head's items within one XCD
};

int launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream);

struct PrologueArgs {
  void* q_out;
  const void* q;
  const void* k;
  const void* v;
  const void* q_weight;
  const void* k_weight;
  const float* cos_sin;
  const int32_t* positions;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int num_tokens;
  int num_q_heads;
  int num_kv_heads;
  int max_position;
  float eps;
  long long num_slots;
};

int launch_store_prologue(const PrologueArgs& a, int head_dim, int dtype_bf16,
                          hipStream_t stream);

}  // namespace pa
