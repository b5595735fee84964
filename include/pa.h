/*
 * pa.h -- C ABI of libpa: attention over a paged KV cache on MI355X (gfx950).
 *
 * Three calls form one attention step of an LLM engine that keeps K/V in a
 * block pool ("nano-vLLM Part 4: Whole-Engine Data Flow, Benchmarks, and the
 * Gap to vLLM V1", section 3, prefill/decode table; "mini-vLLM", project
 * summary):
 *
 *   pa_store_kv        write the new tokens' K/V rows into their pool slots;
 *   pa_decode          one query token per sequence attends to its cached
 *                      history, read through the sequence's block table;
 *   pa_prefill_varlen  packed prompts (boundaries in cu_seqlens) attend
 *                      causally; with cu_seqlens_k > cu_seqlens_q the extra
 *                      keys are a cached prefix (prefix-cache hit).
 *   pa_qk_norm_rope_store  the store with its prologue fused: per-head RMS
 *                      norm and rotary embedding of queries and keys.
 *
 * Data model, shared by every call:
 *   K pool, V pool   [num_blocks, block_size, num_kv_heads, head_dim], row-major,
 *                    two separate allocations of the same dtype;
 *   block_tables     int32 [num_seqs, max_blocks_per_seq], row-major: physical
 *                    block IDs of each sequence in logical order ("nano-vLLM
 *                    Part 4", section 2: a table holds IDs, not K/V);
 *   logical token j of sequence b lives at block block_tables[b][j / block_size],
 *   offset j % block_size; its slot is that block * block_size + offset.
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions:
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing and keeps no pointer after it returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Return values report argument validation and launch
 *     errors only; kernel results are ready when the stream is.
 *   - dtype: PA_DTYPE_F32 (0) or PA_DTYPE_BF16 (1).  q, k, v, both pools and
 *     out share it; accumulation is fp32; outputs are rounded to dtype with
 *     round-to-nearest-even.
 *   - Host integers (max_context_len, max_seqlen_q/k, total_q) size the launch
 *     grid, so no device-to-host copy is needed.
 *   - Device-resident preconditions are not checked on the device:
 *     slots < num_blocks * block_size and distinct; block IDs in
 *     [0, num_blocks); 1 <= context_lens[b] <= max_context_len;
 *     cu_seqlens_* start at 0 and are non-decreasing; 0 <= Lq <= Lk per
 *     sequence.  Kernels clamp block IDs and lengths so that a violated
 *     precondition never reads or writes outside the caller's buffers; the
 *     result is then unspecified.  With the environment variable PA_CHECK=1
 *     the library copies the index arrays to the host, validates them and
 *     returns PA_E_INVAL on a violation (this synchronises the stream).
 *   - scale (the softmax temperature applied to q.k) must be finite and > 0.
 *   - Outputs must not alias inputs; k/v must not alias the pools.
 *   - pa_decode and pa_prefill_varlen move element rows in 16-byte pieces:
 *     out, q and both pools must be 16-byte aligned (else PA_E_INVAL).
 *   - The library keeps no state between calls apart from a per-device cache
 *     of each persistent kernel's occupancy, filled on first use (threads
 *     that fill it together store the same value).  Calls on different
 *     streams may overlap as long as each has a workspace of its own.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_E_INVAL = -1,        /* null pointer, bad size, Hq % Hkv != 0, bad index data */
  PA_E_UNSUPPORTED = -2,  /* head_dim or dtype outside what the kernels cover */
  PA_E_WORKSPACE = -3,    /* workspace too small */
  PA_E_HIP = -4,          /* HIP runtime error while launching */
  PA_E_NOMEM = -5         /* block manager: not enough free blocks (nothing changed) */
};

enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

/*
 * Store: for each token t in [0, num_tokens) with s = slot_mapping[t] >= 0,
 * copy row k[t] (num_kv_heads * head_dim elements) to k_cache slot s, i.e.
 * element [s / block_size][s % block_size][:][:], and v[t] to v_cache slot s.
 * A negative slot means "skip this row" (padding).  Rows are copied bit for
 * bit.  Any head_dim >= 1 is accepted.
 *   k, v          [num_tokens, num_kv_heads, head_dim], contiguous
 *   k_cache, v_cache  the pools (modified in place)
 *   slot_mapping  int32 [num_tokens]
 * ("nano-vLLM Part 4", section 3: K/V is written for every new prompt token in
 * prefill and for one token per sequence in decode; the smzdm Nano-vLLM
 * walk-through, model implementation details: the store puts K and V at their
 * physical position.)  num_tokens == 0 is a no-op (pointers may be NULL).
 * Slots >= num_blocks * block_size are skipped rather than written.
 */
int pa_store_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, int32_t num_blocks, int32_t block_size, int32_t dtype,
                void* stream);

/* Tokens per split-context partition of pa_decode (fixed, so that a row's
 * result depends only on its own tokens). */
#define PA_DECODE_PARTITION_TOKENS 512

/*
 * Bytes of workspace pa_decode may need: a 256-byte work counter, then fp32
 * split-context partial results (unnormalised output, running max and sum
 * per sequence, query head and 512-token context partition, for
 * ceil(max_context_len / 512) partitions).  Depends only on these sizes.
 * 0 when any size is <= 0.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len);

/*
 * Decode: out[b, h, :] = softmax_j(scale * <q[b, h], K_b[j, h / G]>) . V_b[j, h / G]
 * over the context_lens[b] tokens of sequence b (which include the token just
 * stored), where K_b / V_b are gathered through block_tables[b] and
 * G = num_q_heads / num_kv_heads ("mini-vLLM", project summary: in decode each
 * sequence adds one query row, scored against that sequence's stored history;
 * "nano-vLLM Part 4", section 3: decode attention runs over the cached history).
 *   out, q        [num_seqs, num_q_heads, head_dim]
 *   context_lens  int32 [num_seqs]
 *   head_dim      64 or 128
 *   max_context_len  host upper bound of context_lens (sizes the grid)
 *   bf16 query groups of 4 or more heads (G >= 4) run on the matrix cores,
 *   other shapes and fp32 on the vector ALUs; the choice depends only on
 *   (dtype, head_dim, G), so a row's result never depends on the batch, the
 *   block size or the physical block IDs.
 *   workspace     device memory of at least
 *                 pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 *                 max_context_len) bytes, 256-byte aligned.  Its first 256
 *                 bytes hold a work counter that must be zero before the
 *                 first call that uses this memory as a workspace (clear it
 *                 once, e.g. with hipMemset); every call leaves it zero
 *                 again, so a workspace can be reused by any later call on
 *                 the same stream.  The rest is scratch.  Calls that run
 *                 concurrently need workspaces of their own.  Only batches
 *                 with a context longer than 512 tokens use it (else it
 *                 may be NULL).  With PA_CHECK=1 a non-zero counter is
 *                 rejected with PA_E_WORKSPACE.
 * num_seqs == 0 is a no-op.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
              int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
              float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments and results are those of pa_decode
 * (same kernels, same bits).  The split-context workspace is a device array
 * inside the library, PA_NOALLOC_SCRATCH_BYTES bytes per GPU, created when
 * the library is loaded on that GPU and held until the process ends; the
 * call allocates nothing.  Its work counter is cleared on `stream` by a small
 * kernel (no memset node) before each call that uses it.
 *   Limit: pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 *   max_context_len) must not exceed PA_NOALLOC_SCRATCH_BYTES, else
 *   PA_E_WORKSPACE (nothing enqueued).  Batches whose contexts fit one
 *   512-token partition use no workspace and have no limit.
 *   Every call on a GPU shares that GPU's array: calls that may overlap on
 *   one GPU (different streams, or several host threads) race and give
 *   undefined results; serialise them, or use pa_decode with a workspace
 *   per stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                      int32_t dtype, void* stream);

/* Workspace bytes pa_prefill_varlen takes (its work counter). */
#define PA_PREFILL_WORKSPACE_BYTES 256

/*
 * Varlen causal prefill.  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) (Lq of them) and Lk =
 * cu_seqlens_k[b+1] - cu_seqlens_k[b] keys, all read from the pools through
 * block_tables[b] (store the new rows with pa_store_kv first).  The new rows
 * are the last Lq tokens of the sequence, so row i attends to keys
 * 0 .. (Lk - Lq) + i ("mini-vLLM", project summary: a row of a packed
 * prompt sees its own prompt up to its own position; the smzdm Nano-vLLM walk-through, model
 * implementation details: cu_seqlens_k > cu_seqlens_q marks a prefix-cache
 * hit).
 *   out, q        [total_q, num_q_heads, head_dim] packed
 *   cu_seqlens_q, cu_seqlens_k  int32 [num_seqs + 1]
 *   max_seqlen_q, max_seqlen_k  host upper bounds of Lq and Lk
 *   head_dim      64 or 128
 *   workspace     NULL, or device memory of at least PA_PREFILL_WORKSPACE_BYTES
 *                 bytes, 256-byte aligned, holding work counters: all of it
 *                 must be zero before the first call that uses the memory
 *                 (every call leaves it zero).  With it, the query tiles left
 *                 after each workgroup's first go to whichever workgroup is
 *                 free (within groups of workgroups that share an XCD, each
 *                 group taking the tiles of its own KV heads, when the head
 *                 count allows); without it they are dealt in a fixed order.
 *                 Results are bitwise the same either way.  Calls that run
 *                 concurrently need workspaces of their own.  PA_E_WORKSPACE
 *                 if too small, or (with PA_CHECK=1) if a counter is not
 *                 zero.
 * bf16 runs on the matrix cores; fp32 runs on the vector ALUs (and ignores
 * the workspace).
 * num_seqs == 0 or total_q == 0 is a no-op.
 */
int pa_prefill_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                      int32_t block_size, int32_t max_blocks_per_seq, float scale,
                      int32_t dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Store prologue: normalise and rotate the new tokens' queries and keys, then
 * store keys and values -- the step between the projections and
 * pa_store_kv's plain copy, in one pass.  For each token t and each head row
 * x (D = head_dim elements) of q[t] and k[t]:
 *     y_i = x_i / sqrt(mean_j(x_j^2) + eps) * w_i      (w = q_weight or k_weight)
 *     for i < D/2, c = cos_sin[p][i], s = cos_sin[p][D/2 + i], p = positions[t]:
 *         out_i = y_i * c - y_{i+D/2} * s,   out_{i+D/2} = y_{i+D/2} * c + y_i * s
 * (the smzdm Nano-vLLM walk-through, model implementation details: Qwen3
 * normalises queries and keys per head; "mini-vLLM", project summary: rotary
 * embeddings).  Normalised, rotated queries go to q_out (which may be q
 * itself); normalised, rotated keys and the raw values go to pool slot
 * slot_mapping[t] as pa_store_kv does (negative slots are skipped).
 * Arithmetic is fp32; results are rounded once to dtype (round to nearest
 * even).
 *   q, q_out      [num_tokens, num_q_heads, head_dim]
 *   k, v          [num_tokens, num_kv_heads, head_dim]
 *   q_weight, k_weight  [head_dim] gains, same dtype
 *   cos_sin       float32 [max_position, head_dim]: cos in the first half of
 *                 each row, sin in the second (the model's rotary table)
 *   positions     int32 [num_tokens], each in [0, max_position) (clamped into
 *                 range on the device; PA_CHECK=1 rejects violations)
 *   head_dim      64 or 128; every element array and cos_sin 16-byte aligned
 *   eps           finite, >= 0
 * num_tokens == 0 is a no-op.
 */
int pa_qk_norm_rope_store(void* q_out, const void* q, const void* k, const void* v,
                          const void* q_weight, const void* k_weight, const float* cos_sin,
                          const int32_t* positions, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                          int32_t block_size, int32_t max_position, float eps, int32_t dtype,
                          void* stream);

/*
 * Host block manager: the CPU bookkeeping that produces the kernels' paging
 * inputs ("nano-vLLM Part 4", section 1: block IDs, reference counts and
 * prefix-hash metadata live on the CPU; "mini-vLLM", features list: blocks
 * come from a pool fixed at start-up, taken and returned in constant time,
 * and each sequence keeps a table of the blocks it owns).  Full blocks are registered under their token content chained
 * with their predecessor, so a sequence starting with the same full blocks
 * shares them (reference counts) -- an exact full-block prefix cache (smzdm
 * Nano-vLLM walk-through, scheduling and memory).  A freed block keeps its
 * registration until the free list (first in, first out) hands it out again,
 * so a preempted sequence that is allocated again finds its computed blocks.
 * Sequences are named by caller-chosen 64-bit IDs.  The object is not
 * thread-safe; it never touches the GPU.  Block IDs are indices into the
 * pools given to the kernels (num_blocks must match).
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks blocks of block_size tokens; NULL on bad sizes. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);
/* Blocks on the free list (cached blocks with no user count as free). */
int32_t pa_bm_num_free(const pa_block_manager* m);
/* Blocks for a new sequence's prompt tokens[0 .. num_tokens): reuses cached
 * full blocks from the start while they match, then takes fresh ones.
 * *num_cached_tokens = the leading tokens whose K/V the pool already holds
 * (at most num_tokens - 1: the last token is always recomputed).  Returns
 * PA_E_NOMEM (and changes nothing) when the pool is short, PA_E_INVAL for a
 * known seq_id or an empty prompt. */
int pa_bm_allocate(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                   int32_t num_tokens, int32_t* num_cached_tokens);
/* Append one decoded token; *slot = its pool slot (block * block_size +
 * offset), taking a new block when the token opens one (PA_E_NOMEM if none
 * is free) and registering the block when the token fills it. */
int pa_bm_append(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot);
/* Release a sequence (finished or preempted): each block's count drops, and
 * blocks reaching zero go to the free list, last block first. */
int pa_bm_free(pa_block_manager* m, int64_t seq_id);
/* The sequence's block table; *num_blocks gets its length (PA_E_INVAL if it
 * exceeds capacity; out may be NULL to ask for the length). */
int pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* out,
                      int32_t capacity, int32_t* num_blocks);
/* Token count and cached-prefix length of a sequence. */
int pa_bm_seq_info(const pa_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                   int32_t* num_cached_tokens);
/* Slots of tokens [first, first + count) of a sequence (the slot mapping of
 * a step's new tokens). */
int pa_bm_slots(const pa_block_manager* m, int64_t seq_id, int32_t first, int32_t count,
                int32_t* slots);

/* Batched forms for a scheduler's step (one call per step instead of one
 * per sequence).  All buffers are host memory owned by the caller; block
 * table rows are padded with block 0 past each sequence's blocks.
 *
 * Append tokens[i] to seq_ids[i] for i in order.  Stops at the first
 * sequence whose new token needs a block when none is free: returns
 * PA_E_NOMEM with *num_done = the appends made (kept; slots[0 .. num_done)
 * valid), so the caller can preempt and continue from there.  PA_E_INVAL
 * for an unknown ID, with *num_done likewise. */
int pa_bm_append_batch(pa_block_manager* m, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t num_seqs, int32_t* slots, int32_t* num_done);
/* Decode-step inputs: block_tables [num_seqs, table_width], context_lens
 * [num_seqs] (token counts), *max_context_len.  PA_E_INVAL (nothing
 * written) for an unknown ID or a table wider than table_width. */
int pa_bm_plan_decode(const pa_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                      int32_t table_width, int32_t* block_tables, int32_t* context_lens,
                      int32_t* max_context_len);
/* Prefill-step inputs for sequences just allocated: the query rows of
 * sequence i are its tokens past the cached prefix.  block_tables
 * [num_seqs, table_width]; cu_seqlens_q / cu_seqlens_k [num_seqs + 1];
 * slot_mapping [sum of query rows] (the store's slots, in packed row order);
 * *max_seqlen_q / *max_seqlen_k.  PA_E_INVAL (nothing written) for an
 * unknown ID, a table wider than table_width or more query rows than
 * slot_capacity. */
int pa_bm_plan_prefill(const pa_block_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t table_width, int32_t* block_tables, int32_t* cu_seqlens_q,
                       int32_t* cu_seqlens_k, int32_t* slot_mapping, int32_t slot_capacity,
                       int32_t* max_seqlen_q, int32_t* max_seqlen_k);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
