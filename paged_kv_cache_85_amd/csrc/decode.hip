// Decode attention over a paged KV cache on the vector ALUs, split over the
// context with an online softmax.
//
// A decode step scores one new query row per sequence against the whole
// stored history of that sequence ("mini-vLLM", project summary), read
// through the sequence's block table ("nano-vLLM Part 4", section 3: decode
// attention over the cached history).  The work is HBM-bound (about 2 FLOP
// per byte of bf16 KV at a query group of 2), so the kernels are organised
// around the memory stream, not the matrix cores:
//
//  * the unit of work is an item = (sequence, 512-token context partition,
//    KV head); the query heads of the KV head's group (up to HG of them)
//    share every K/V row loaded, so each KV byte is read once per group;
//  * one wave folds an item in stages of SUB tokens; each lane loads 16
//    contiguous bytes of a token's head row, LPR lanes cover the row and RPS
//    rows load per instruction (fully used 16-byte accesses);
//  * q.k partial dot products are reduced across the LPR lanes of a row with
//    DPP (quad permutes and row mirrors), which leaves every lane of the row
//    holding the full score, so probabilities need no broadcast;
//  * each lane row keeps its own running max / sum / output (an independent
//    online softmax), merged across rows once per item;
//  * an item of a sequence with several partitions writes an unnormalised
//    partial (output, max, sum) to the workspace; a small combine kernel
//    rescales and sums them.  A one-partition sequence is finished in place.
//    The partition size is fixed, so a row's arithmetic depends only on its
//    own tokens: results are bitwise independent of the batch, the physical
//    block IDs and the block size.
//
// Large power-of-two blocks (>= 64 tokens; 256 in the Qwen3 workloads) run a
// persistent kernel: one wave per SIMD walks an equal, contiguous
// share of all items, and a ring of register stages keeps NBUF - 1 stages in
// flight across item boundaries, so the memory stream never drains between
// items and no launch slot is spent on empty partitions.  Each stage is read
// through a raw buffer descriptor that covers exactly its valid rows (rows
// past the end read zero).  Other block sizes, and the fp32 prefill rows
// ("varlen": row i of a sequence with Lq new and Lk total tokens is a decode
// over its first Lk - Lq + i + 1 keys), use one wave per item.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

struct ElemF32 {
  typedef float storage;
  static constexpr int EPL = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static __forceinline__ void store(storage* p, float x) { *p = x; }
};

struct ElemBF16 {
  typedef uint16_t storage;
  static constexpr int EPL = 8;
  __device__ static __forceinline__ void widen(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x);
    f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y);
    f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z);
    f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w);
    f[7] = bf16_hi(u.w);
  }
  __device__ static __forceinline__ void store(storage* p, float x) {
    *reinterpret_cast<__bf16*>(p) = (__bf16)x;
  }
};

#ifndef PA_DECODE_STAGE_STEPS
#define PA_DECODE_STAGE_STEPS 4
#endif
#ifndef PA_DECODE_STAGES
#define PA_DECODE_STAGES 3
#endif
constexpr int kStageSteps = PA_DECODE_STAGE_STEPS;  // load steps per stage
constexpr int kStages = PA_DECODE_STAGES;           // register stages in the ring

// Raw buffer descriptor (GFX9 family: dword3 = 0x00020000) over `bytes`
// bytes at `base`; loads at offsets past the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Decode reads every key/value row once per call, so its loads carry the
// non-temporal cache policy (gfx940-family cache-policy bit NT = 2), which
// lets them stream past the caches.  A streaming probe of this access
// pattern (256-byte rows at the pool's token stride, three 8 KB register
// stages per wave, two waves per SIMD) reads 6.48 TB/s with it and 5.89 TB/s
// without.  Rows that other query rows read again (the fp32 varlen path)
// keep the default policy, and so do the bf16 prefill tiles: with it the
// prefill kernel runs 15-20 % slower, its tiles being re-read through L2.
constexpr int kStreamPolicy = 2;

template <bool STREAM>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, STREAM ? kStreamPolicy : 0));
}

template <bool STREAM>
__device__ __forceinline__ uint4 load16(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* v = reinterpret_cast<const u32x4*>(p);
  if constexpr (STREAM) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(v));
  else return __builtin_bit_cast(uint4, *v);
}

// Online-softmax state of one wave for HG query heads (lane = row r of RPS,
// column c of LPR).
template <typename E, int D, int HG>
struct RowFold {
  static constexpr int EPL = E::EPL;
  static constexpr int LPR = D / EPL;  // lanes per K/V head row
  static constexpr int RPS = 64 / LPR;  // token rows per load instruction
  static constexpr int SS = kStageSteps;
  static constexpr int SUB = SS * RPS;  // tokens per stage
  typedef typename E::storage T;

  float qf[HG][EPL];  // queries pre-multiplied by scale * log2(e)
  float m[HG], l[HG], o[HG][EPL];

  __device__ __forceinline__ void set_q(const uint4 (&raw)[HG], float scale_log2) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      E::widen(raw[h], qf[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] *= scale_log2;
    }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      m[h] = kNegBig;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }
  }

  // Fold one stage (tokens t0 .. t0 + SUB - 1, of which those < tok_end
  // count).  Rows past the end hold zeros or a copy of a valid row: finite
  // values whose scores are masked here, so they add nothing.
  __device__ __forceinline__ void fold(const uint4 (&kr)[SS], const uint4 (&vr)[SS], int t0,
                                       int tok_end, int r) {
    float sc[HG][SS];
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      float kf[EPL];
      E::widen(kr[s], kf);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
        sc[h][s] = acc;
      }
    }
#pragma unroll
    for (int s = 0; s < SS; ++s)
#pragma unroll
      for (int h = 0; h < HG; ++h) sc[h][s] = group_sum<LPR>(sc[h][s]);
    if (t0 + SUB > tok_end) {
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const bool valid = t0 + s * RPS + r < tok_end;
#pragma unroll
        for (int h = 0; h < HG; ++h) sc[h][s] = valid ? sc[h][s] : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float mx = sc[h][0];
#pragma unroll
      for (int s = 1; s < SS; ++s) mx = fmaxf(mx, sc[h][s]);
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      float lsum = l[h] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const float pr = fast_exp2(sc[h][s] - mn);
        lsum += pr;
        sc[h][s] = pr;
      }
      l[h] = lsum;
    }
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      float vf[EPL];
      E::widen(vr[s], vf);
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(sc[h][s], vf[e], o[h][e]);
    }
  }

  // Max / sum over the RPS lane rows holding the same column c (lanes c,
  // c + LPR, ...): pairwise steps at distances LPR, 2 LPR, ... 32.
  __device__ static __forceinline__ float rows_max(float x) {
    if constexpr (LPR <= 8) x = xor_max<8>(x);
    if constexpr (LPR <= 16) x = xor_max<16>(x);
    return xor_max<32>(x);
  }
  __device__ static __forceinline__ float rows_sum(float x) {
    if constexpr (LPR <= 8) x = xor_sum<8>(x);
    if constexpr (LPR <= 16) x = xor_sum<16>(x);
    return xor_sum<32>(x);
  }

  // Merge the RPS independent row states (lanes c, c + LPR, ...) and write
  // the item: normalised output when the sequence has one partition, else an
  // unnormalised partial.  Lanes of row 0 hold the merged state.
  __device__ __forceinline__ void finish(const RowAttnArgs& a, long oh0, int nparts, int p,
                                         int c, int r) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float M = rows_max(m[h]);
      const float wgt = fast_exp2(m[h] - M);
      const float lw = rows_sum(l[h] * wgt);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = rows_sum(o[h][e] * wgt);
      m[h] = M;
      l[h] = lw;
    }
    if (r != 0) return;
    T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const long oh = oh0 + h;
      if (nparts == 1) {
        const float inv = 1.f / l[h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) E::store(out + oh * D + c * EPL + e, o[h][e] * inv);
      } else {
        float* po = a.ws_o + (oh * a.max_parts + p) * D + c * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<float4*>(po + e) =
              make_float4(o[h][e], o[h][e + 1], o[h][e + 2], o[h][e + 3]);
        if (c == 0) {
          a.ws_ml[(oh * a.max_parts + p) * 2] = m[h];
          a.ws_ml[(oh * a.max_parts + p) * 2 + 1] = l[h];
        }
      }
    }
  }
};


// ---------------------------------------------------------------- one wave per item
//
// BIG: power-of-two blocks of >= 64 tokens (a stage never straddles a block).
// Otherwise decode stages its partition's block IDs in LDS (one read at the
// start, so lookups never wait behind the K/V stream) and varlen rows read
// the table per lane.
template <typename E, int D, int HG, bool VARLEN, bool BIG>
__global__ __launch_bounds__(64) void row_attn_kernel(RowAttnArgs a) {
  typedef RowFold<E, D, HG> F;
  typedef typename E::storage T;
  constexpr int EPL = F::EPL, LPR = F::LPR, RPS = F::RPS, SS = F::SS, SUB = F::SUB;
  constexpr int NBUF = kStages;

  const int lane = threadIdx.x;
  const int c = lane % LPR;
  const int r = lane / LPR;

  // blockIdx.x = (row * max_parts + p) * Y + y, Y = kv heads * head chunks
  const int Y = a.num_kv_heads * a.head_chunks;
  int x = blockIdx.x;
  const int y = x % Y;
  x /= Y;
  const int p = x % a.max_parts;
  const int row = x / a.max_parts;
  const int g = y / a.head_chunks;
  const int h0 = g * a.group + (y % a.head_chunks) * HG;

  int b, L;
  if constexpr (!VARLEN) {
    b = row;
    L = min(a.context_lens[b], a.max_context);
  } else {
    int lo = 0, hi = a.num_seqs;  // cu_q[lo] <= row < cu_q[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid;
    }
    b = lo;
    const int i = row - a.cu_seqlens_q[b];
    const int lq = a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b];
    const int lk = min(a.cu_seqlens_k[b + 1] - a.cu_seqlens_k[b], a.max_context);
    L = min(lk - lq + i + 1, lk);
  }

  if (L <= 0) {  // violated precondition: define the output as zeros
    if (p == 0)
      for (int idx = lane; idx < HG * D; idx += 64)
        E::store(reinterpret_cast<T*>(a.out) + ((long)row * a.num_q_heads + h0) * D + idx, 0.f);
    return;
  }
  const int nparts = num_parts(L, a.part_tokens);
  if (p >= nparts) return;
  const int tok_begin = p * a.part_tokens;
  const int tok_end = min(L, tok_begin + a.part_tokens);
  const int32_t* bt = a.block_tables + (long)b * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nb = a.num_blocks;

  constexpr bool kLdsTable = !BIG && !VARLEN;
  // Blocks of one decode partition: at most its token count (block size 1).
  constexpr int kMaxTable = kLdsTable ? kDecodePartition : 1;
  static_assert(!kLdsTable || kDecodePartition % 64 == 0, "partition size");
  __shared__ int s_bt[kMaxTable];
  int first_blk = 0;
  if constexpr (kLdsTable) {
    first_blk = bs_log2 >= 0 ? (tok_begin >> bs_log2) : tok_begin / bs;
    const int last_blk = bs_log2 >= 0 ? ((tok_end - 1) >> bs_log2) : (tok_end - 1) / bs;
    for (int i = lane; i <= last_blk - first_blk && i < kMaxTable; i += 64)
      s_bt[i] = clamp_block(bt[first_blk + i], nb);
    __syncthreads();
  }

  F st;
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((long)row * a.num_q_heads + h0) * D +
                  c * EPL;
    uint4 raw[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) raw[h] = *reinterpret_cast<const uint4*>(qp + h * D);
    st.set_q(raw, a.scale_log2);
  }
  st.reset();

  const T* kc = reinterpret_cast<const T*>(a.k_cache);
  const T* vc = reinterpret_cast<const T*>(a.v_cache);
  const int slot_elems = a.num_kv_heads * D;
  const int head_off = g * D + c * EPL;
  const unsigned row_bytes = (unsigned)slot_elems * (unsigned)sizeof(T);
  unsigned big_off[BIG ? SS : 1];
  if constexpr (BIG) {
#pragma unroll
    for (int s = 0; s < SS; ++s)
      big_off[s] = (unsigned)(s * RPS + r) * row_bytes + (unsigned)(c * EPL * sizeof(T));
  }

  auto load = [&](uint4 (&kr)[SS], uint4 (&vr)[SS], int t0) {
    const int nvalid = tok_end - t0;  // >= 1
    if constexpr (BIG) {
      const int blk = clamp_block(bt[t0 >> bs_log2], nb);
      const long base = (((long)blk << bs_log2) + (t0 & (bs - 1))) * slot_elems + (long)g * D;
      const unsigned bytes = (unsigned)min(nvalid, SUB) * row_bytes;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + base, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + base, bytes);
#pragma unroll
      for (int s = 0; s < SS; ++s) kr[s] = buffer_load16<!VARLEN>(rk, big_off[s]);
#pragma unroll
      for (int s = 0; s < SS; ++s) vr[s] = buffer_load16<!VARLEN>(rv, big_off[s]);
    } else {
      // Rows past the end read the last valid token instead (a written row).
      long off[SS];
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const int j = t0 + min(s * RPS + r, nvalid - 1);
        int blk, in_blk;
        if (bs_log2 >= 0) {
          blk = j >> bs_log2;
          in_blk = j & (bs - 1);
        } else {
          blk = j / bs;
          in_blk = j - blk * bs;
        }
        if constexpr (kLdsTable) blk = s_bt[blk - first_blk];
        else blk = clamp_block(bt[blk], nb);
        off[s] = ((long)blk * bs + in_blk) * slot_elems + head_off;
      }
#pragma unroll
      for (int s = 0; s < SS; ++s) kr[s] = load16<!VARLEN>(kc + off[s]);
#pragma unroll
      for (int s = 0; s < SS; ++s) vr[s] = load16<!VARLEN>(vc + off[s]);
    }
  };

  // A ring of NBUF register stages: NBUF - 1 stages are in flight while one
  // is folded in.  Prefetches are unconditional (past the end they re-read
  // the last stage, which is cached) so the compiler can count outstanding
  // loads exactly; sched_barrier keeps each prefetch above the fold.
  uint4 kbuf[NBUF][SS], vbuf[NBUF][SS];
  const int last_t0 = tok_begin + ((tok_end - tok_begin - 1) / SUB) * SUB;
  int t0 = tok_begin;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) load(kbuf[i], vbuf[i], min(t0 + i * SUB, last_t0));
  for (;;) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      load(kbuf[(i + NBUF - 1) % NBUF], vbuf[(i + NBUF - 1) % NBUF],
           min(t0 + (NBUF - 1) * SUB, last_t0));
      __builtin_amdgcn_sched_barrier(0);
      st.fold(kbuf[i], vbuf[i], t0, tok_end, r);
      if (t0 >= last_t0) goto folded;
      t0 += SUB;
    }
  }
folded:
  st.finish(a, (long)row * a.num_q_heads + h0, nparts, p, c, r);
}

// ---------------------------------------------------------------- persistent decode
//
// Items are numbered by a code: [0, n_full) are the full partitions (P
// tokens) in (sequence b, head chunk y, partition p) order, p fastest;
// [n_full, n_full + n_partial) are the partial last partitions, largest size
// class first, then (b, y).
//
// Every wave first folds an equal-count contiguous run of full partitions
// (consecutive items mostly share their query rows).  Waves on a loaded chip
// do not stream at equal rates (the XCDs and the slots within a CU differ),
// so a static deal of everything leaves the last waves running alone.  With a
// ticket counter (the decode workspace holds one), the static runs cover only
// part of the full partitions; the rest, then the partials, largest first,
// are handed out one ticket at a time to whichever wave is free.  Each wave
// draws until a draw comes back past the last item, so a launch of W waves
// makes exactly W such draws; the wave that draws the very last value knows
// that no one will touch the counter again and puts it back to zero, so
// every call leaves the counter as it found it (zero).  Without a
// counter (one-partition batches: no workspace) the partials are dealt in a
// snake over size classes that starts at the waves with the shorter static
// run.  Which wave folds an item does not change the item's arithmetic.

constexpr int kSizeClasses = 16;
constexpr int kMaxDealSeqs = 4096;  // per-sequence deal tables kept in LDS up to this batch
#ifndef PA_DECODE_STATIC_PCT
#define PA_DECODE_STATIC_PCT 60
#endif
constexpr int kStaticPct = PA_DECODE_STATIC_PCT;  // full partitions dealt statically (percent)

// Integer DPP step: x of the lane selected by the GFX9 DPP control CTRL
// (rows outside ROWS, and lanes whose source lies outside their row, read 0).
template <int CTRL, int ROWS = 0xF, bool BC = true>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, BC);
}

// Sum of x over the wave, register to register: the two quad permutes and
// the two mirrors sum each 16-lane row, the lane swaps add rows 16 and 32
// apart (no LDS round trips).
__device__ __forceinline__ int wave_sum(int x) {
  x += dpp_i32<DPP_QUAD_1032>(x);
  x += dpp_i32<DPP_QUAD_2301>(x);
  x += dpp_i32<DPP_ROW_HALF_MIRROR>(x);
  x += dpp_i32<DPP_ROW_MIRROR>(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = (int)(r16[0] + r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(r32[0] + r32[1]);
}

// Inclusive prefix sum over the wave: shifts by 1, 2, 4 and 8 lanes inside
// each 16-lane row, then lane 15 of a row is added to the next row (rows 1
// and 3) and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_scan(int x) {
  x += dpp_i32<0x111>(x);        // row_shr:1
  x += dpp_i32<0x112>(x);        // row_shr:2
  x += dpp_i32<0x114>(x);        // row_shr:4
  x += dpp_i32<0x118>(x);        // row_shr:8
  x += dpp_i32<0x142, 0xA, false>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_i32<0x143, 0xC, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

struct ItemCursor {
  int b, p, y;     // sequence, partition, head chunk
  int L;           // context length of b
  int t0, end;     // current stage start, end of the item's tokens
};

// Wave-uniform description of the deal.  Per-sequence tables live in LDS, so
// that finding an item never issues a vector load (it would wait behind the
// K/V stream).
struct Deal {
  int B, Y, P, W, w;
  long n_full;      // full partitions
  int n_partial;    // partial partitions
  bool in_lds;      // the LDS tables below hold the batch
};
__shared__ uint8_t s_deal_cls[kMaxDealSeqs];    // size class of each sequence's partial partition
__shared__ uint16_t s_deal_full[kMaxDealSeqs];  // full partitions of each sequence
__shared__ int s_deal_chunk[kMaxDealSeqs / 64];  // full items before each 64-sequence chunk
__shared__ int s_deal_cnt[kSizeClasses];        // partial items per class, largest first

// `lens` is the same array as a.context_lens, passed as a __restrict__
// kernel argument: the kernel never writes it, so its reads can be scalar
// loads (counted apart from the K/V stream) rather than vector loads.
__device__ __forceinline__ int seq_len(const RowAttnArgs& a, const int32_t* __restrict__ lens,
                                       int b) {
  return b < a.num_rows ? min(lens[b], a.max_context) : 1;
}

__device__ __forceinline__ int full_parts(int L, int P) { return L > 0 ? L / P : 0; }

// Size class of a sequence's partial last partition (0: none).
__device__ __forceinline__ int tail_class(int L, int P) {
  const int t = L > 0 ? L - (L / P) * P : 0;
  return t > 0 ? (t * kSizeClasses + P - 1) / P : 0;
}

__device__ __forceinline__ void cursor_begin(ItemCursor& k, int P) {
  k.t0 = k.p * P;
  k.end = min(k.L, k.t0 + P);
}

// Full partition of rank `target`, from the lengths (before the stream starts
// or when the batch is too large for the LDS tables).
__device__ __forceinline__ void seek_full_scan(ItemCursor& k, long target, const Deal& d,
                                               const RowAttnArgs& a,
                                               const int32_t* __restrict__ lens, int lane) {
  long acc = 0;
  k.b = d.B;
  int off = 0;
  for (int base = 0; base < d.B; base += 64) {
    const int b = base + lane;
    const int ni = b < d.B ? d.Y * full_parts(min(lens[b], a.max_context), d.P) : 0;
    const int incl = wave_scan(ni);
    const int chunk = __builtin_amdgcn_readlane(incl, 63);
    if (acc + chunk > target) {
      const unsigned long long hit = __ballot(acc + incl > target);
      const int l0 = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
      const int excl = __builtin_amdgcn_readlane(incl - ni, l0);
      k.b = base + l0;
      off = (int)(target - acc - excl);
      break;
    }
    acc += chunk;
  }
  k.b = __builtin_amdgcn_readfirstlane(k.b);
  k.L = seq_len(a, lens, k.b);
  const int nf = max(full_parts(k.L, d.P), 1);
  off = __builtin_amdgcn_readfirstlane(off);
  k.y = off / nf;
  k.p = off % nf;
  cursor_begin(k, d.P);
}

// The same from the LDS tables: one ballot over the chunk prefixes, one scan
// inside the chunk.
__device__ __forceinline__ void seek_full_lds(ItemCursor& k, long target, const Deal& d,
                                              const RowAttnArgs& a,
                                              const int32_t* __restrict__ lens, int lane) {
  const int nchunks = (d.B + 63) >> 6;
  const int t = (int)target;  // n_full < 2^31 whenever the tables are used
  const int pref = lane < nchunks ? s_deal_chunk[lane] : 0x7fffffff;
  const unsigned long long le = __ballot(pref <= t);
  const int ch = __builtin_amdgcn_readfirstlane(63 - (int)__builtin_clzll(le));
  const int cbase = __builtin_amdgcn_readlane(pref, ch);
  const int b = ch * 64 + lane;
  const int ni = b < d.B ? d.Y * (int)s_deal_full[b] : 0;
  const int incl = wave_scan(ni);
  const unsigned long long hit = __ballot(cbase + incl > t);
  const int l0 = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
  const int excl = __builtin_amdgcn_readlane(incl - ni, l0);
  k.b = ch * 64 + l0;
  k.L = seq_len(a, lens, k.b);
  const int nf = max(full_parts(k.L, d.P), 1);
  const int off = t - cbase - excl;
  k.y = off / nf;
  k.p = off % nf;
  cursor_begin(k, d.P);
}

__device__ __forceinline__ void next_full(ItemCursor& k, const Deal& d, const RowAttnArgs& a,
                                          const int32_t* __restrict__ lens) {
  if (++k.p >= full_parts(k.L, d.P)) {
    k.p = 0;
    if (++k.y == d.Y) {
      k.y = 0;
      do {
        ++k.b;
        k.L = seq_len(a, lens, k.b);
      } while (full_parts(k.L, d.P) == 0 && k.b < d.B);
    }
  }
  cursor_begin(k, d.P);
}

// Rank of this wave's partial item in round r of the snake.
__device__ __forceinline__ int partial_rank(const Deal& d, int r) {
  return r * d.W + ((r & 1) ? d.w : d.W - 1 - d.w);
}

// Partial item of rank j (size class descending, then (b, y)).
__device__ __forceinline__ void seek_partial(ItemCursor& k, int j, const Deal& d,
                                             const RowAttnArgs& a,
                                             const int32_t* __restrict__ lens, int lane) {
  int c = 1;
  for (int i = 0; i < kSizeClasses; ++i) {
    const int n = __builtin_amdgcn_readfirstlane(s_deal_cnt[i]);
    if (j < n) {
      c = kSizeClasses - i;
      break;
    }
    j -= n;
  }
  const int bi = j / d.Y;
  k.y = j - bi * d.Y;
  k.b = d.B;
  int seen = 0;
  for (int base = 0; base < d.B; base += 64) {
    const int b = base + lane;
    const bool in = b < d.B && (d.in_lds ? (int)s_deal_cls[b]
                                         : tail_class(min(lens[b], a.max_context), d.P)) == c;
    const unsigned long long m = __ballot(in);
    const int n = __popcll(m);
    if (bi < seen + n) {
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
      const unsigned long long sel = __ballot(in && below == bi - seen);
      k.b = base + (int)__builtin_ctzll(sel);
      break;
    }
    seen += n;
  }
  k.b = __builtin_amdgcn_readfirstlane(k.b);
  k.L = seq_len(a, lens, k.b);
  k.p = full_parts(k.L, d.P);  // the partial partition is the last one
  cursor_begin(k, d.P);
}

// Cursor of item `code` (see the numbering above); `prev` is the cursor of
// item code - 1 when the caller has it (then a full item is one step on).
__device__ __forceinline__ void seek_item(ItemCursor& k, long code, bool follows,
                                          const Deal& d, const RowAttnArgs& a,
                                          const int32_t* __restrict__ lens, int lane) {
  if (code < d.n_full) {
    if (follows) next_full(k, d, a, lens);
    else if (d.in_lds) seek_full_lds(k, code, d, a, lens, lane);
    else seek_full_scan(k, code, d, a, lens, lane);
  } else {
    seek_partial(k, (int)(code - d.n_full), d, a, lens, lane);
  }
}

template <typename E, int D, int HG>
__global__ __launch_bounds__(64) void decode_persistent_kernel(
    RowAttnArgs a, const int32_t* __restrict__ lens, const int32_t* __restrict__ tables) {
  typedef RowFold<E, D, HG> F;
  typedef typename E::storage T;
  constexpr int EPL = F::EPL, LPR = F::LPR, RPS = F::RPS, SS = F::SS, SUB = F::SUB;
  constexpr int NBUF = kStages;

  const int lane = threadIdx.x;
  const int c = lane % LPR;
  const int r = lane / LPR;
  Deal d;
  d.B = a.num_rows;
  d.P = a.part_tokens;
  d.Y = a.num_kv_heads * a.head_chunks;
  d.W = gridDim.x;
  d.w = blockIdx.x;
  const int B = d.B, P = d.P, Y = d.Y;

  // Full partitions and partial-partition classes over the batch, and the
  // LDS tables; wave 0 also zeroes rows whose length violates the
  // precondition (no item covers them).  Lengths are read eight chunks of 64
  // at a time, so their loads are in flight together.
  long n_full = 0;
  d.in_lds = B <= kMaxDealSeqs;
  if (lane < kSizeClasses) s_deal_cnt[lane] = 0;
  __syncthreads();
  constexpr int kUnroll = 8;
  for (int base0 = 0; base0 < B; base0 += 64 * kUnroll) {
    int Lr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int b = base0 + u * 64 + lane;
      Lr[u] = b < B ? min(lens[b], a.max_context) : 1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int base = base0 + u * 64;
      if (base >= B) break;
      const int b = base + lane;
      const int L = Lr[u];
      if (d.w == 0 && L <= 0)
        for (int i = 0; i < a.num_q_heads * D; ++i)
          E::store(reinterpret_cast<T*>(a.out) + (long)b * a.num_q_heads * D + i, 0.f);
      const int fp = b < B ? full_parts(L, P) : 0;
      const int cls = b < B ? tail_class(L, P) : 0;
      if (d.in_lds) {
        if (b < B) {
          s_deal_cls[b] = (uint8_t)cls;
          s_deal_full[b] = (uint16_t)min(fp, 0xffff);
        }
        if (lane == 0) s_deal_chunk[base >> 6] = (int)min(n_full, 0x7fffffffL);
      }
      if (cls > 0) atomicAdd(&s_deal_cnt[kSizeClasses - cls], Y);
      n_full += (long)Y * __builtin_amdgcn_readfirstlane(wave_sum(fp));
    }
  }
  __syncthreads();
  const int n_partial =
      __builtin_amdgcn_readfirstlane(wave_sum(lane < kSizeClasses ? s_deal_cnt[lane] : 0));
  d.n_full = n_full;
  d.n_partial = n_partial;
  // The LDS tables serve lookups only while every count fits them.
  d.in_lds = d.in_lds && n_full < 0x7fffffffL && a.max_context / P < 0xffff;
  const bool dyn = a.ticket != nullptr && d.in_lds;
  const long n_items = n_full + n_partial;

  // This wave's static run of full partitions (of the first n_static), then
  // tickets or its share of the partial snake.
  const long n_static = dyn ? n_full * kStaticPct / 100 : n_full;
  const long fa = n_static / d.W, frem = n_static % d.W;
  const long f0 = d.w < frem ? d.w * (fa + 1) : frem * (fa + 1) + (d.w - frem) * fa;
  const int nfull_w = (int)(d.w < frem ? fa + 1 : fa);
  const int rounds = n_partial / d.W, prem = n_partial % d.W;
  const int npart_w =
      dyn ? 0 : rounds + (((rounds & 1) ? d.w : d.W - 1 - d.w) < prem ? 1 : 0);

  // Loader state: its cursor and item code, the static items still to
  // visit after the current one, and the next snake round.  A ticket is
  // taken when the loader reaches the last stage of its last assigned item,
  // one stage before it is needed, so that the item goes to a wave that is
  // about to be free.  (The compiler emits the single-lane draw in a
  // wave-aggregated form that reads its result at once, so the wave waits
  // for the atomic and the stages in flight right there; compiling without
  // that form measured slower.)
  ItemCursor ld;
  long ld_code;
  int ld_full_left = 0, ld_round = 0;
  unsigned tk = 0;
  // The draw that returns this value is the last one of the launch.
  const unsigned last_draw = (unsigned)(n_items - n_static) + (unsigned)d.W - 1u;
  auto past_end = [&](unsigned t) __attribute__((always_inline)) {
    if (t == last_draw && lane == 0)
      __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (nfull_w > 0) {
    ld_full_left = nfull_w - 1;
    ld_code = f0;
    if (d.in_lds) seek_full_lds(ld, f0, d, a, lens, lane);
    else seek_full_scan(ld, f0, d, a, lens, lane);
  } else if (dyn) {
    if (lane == 0) tk = atomicAdd(a.ticket, 1u);
    const unsigned t = __builtin_amdgcn_readfirstlane(tk);
    ld_code = n_static + (long)t;
    if (ld_code >= n_items) {
      past_end(t);
      return;
    }
    seek_item(ld, ld_code, false, d, a, lens, lane);
  } else {
    if (npart_w <= 0) return;
    ld_code = n_full + partial_rank(d, ld_round++);
    seek_partial(ld, (int)(ld_code - n_full), d, a, lens, lane);
  }

  const T* kc = reinterpret_cast<const T*>(a.k_cache);
  const T* vc = reinterpret_cast<const T*>(a.v_cache);
  const int slot_elems = a.num_kv_heads * D;
  const unsigned row_bytes = (unsigned)slot_elems * (unsigned)sizeof(T);
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nb = a.num_blocks;
  unsigned lane_off[SS];
#pragma unroll
  for (int s = 0; s < SS; ++s)
    lane_off[s] = (unsigned)(s * RPS + r) * row_bytes + (unsigned)(c * EPL * sizeof(T));

  // Query rows of an item's HG heads.
  auto load_q = [&](uint4 (&raw)[HG], const ItemCursor& k) __attribute__((always_inline)) {
    const int h0 = (k.y / a.head_chunks) * a.group + (k.y % a.head_chunks) * HG;
    const T* qp = reinterpret_cast<const T*>(a.q) + ((long)k.b * a.num_q_heads + h0) * D +
                  c * EPL;
#pragma unroll
    for (int h = 0; h < HG; ++h) raw[h] = *reinterpret_cast<const uint4*>(qp + h * D);
  };

  // One stage of the loader's item through a descriptor over its valid rows;
  // an item's first stage also brings its query rows.
  auto load = [&](uint4 (&kr)[SS], uint4 (&vr)[SS], uint4 (&qr)[HG], const ItemCursor& k)
      __attribute__((always_inline)) {
    const int g = k.y / a.head_chunks;
    const int blk =
        clamp_block(tables[(long)k.b * a.max_blocks_per_seq + (k.t0 >> bs_log2)], nb);
    const long base = (((long)blk << bs_log2) + (k.t0 & (bs - 1))) * slot_elems + (long)g * D;
    const unsigned bytes = (unsigned)min(k.end - k.t0, SUB) * row_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + base, bytes);
    if (k.t0 == k.p * P) load_q(qr, k);
#pragma unroll
    for (int s = 0; s < SS; ++s) kr[s] = buffer_load16<true>(rk, lane_off[s]);
#pragma unroll
    for (int s = 0; s < SS; ++s) vr[s] = buffer_load16<true>(rv, lane_off[s]);
  };

  // The loader runs NBUF - 1 stages ahead of the fold.  After its last item's
  // last stage it keeps re-reading that stage (cached, unused) with code -1.
  bool ld_done = false;
  auto take_ticket = [&]() __attribute__((always_inline)) {
    if (dyn && ld_full_left == 0 && ld.t0 + SUB >= ld.end && lane == 0)
      tk = atomicAdd(a.ticket, 1u);
  };
  auto ld_advance = [&]() __attribute__((always_inline)) {
    if (ld_done) return;
    if (ld.t0 + SUB < ld.end) {
      ld.t0 += SUB;
      take_ticket();
      return;
    }
    if (ld_full_left > 0) {
      --ld_full_left;
      ++ld_code;
      next_full(ld, d, a, lens);
      take_ticket();
    } else if (dyn) {
      const unsigned t = __builtin_amdgcn_readfirstlane(tk);
      const long next = n_static + (long)t;
      if (next >= n_items) {
        past_end(t);
        ld_done = true;
        return;
      }
      seek_item(ld, next, next == ld_code + 1, d, a, lens, lane);
      ld_code = next;
      take_ticket();
    } else if (ld_round < npart_w) {
      ld_code = n_full + partial_rank(d, ld_round++);
      seek_partial(ld, (int)(ld_code - n_full), d, a, lens, lane);
    } else {
      ld_done = true;
    }
  };

  // Register stages, each tagged with the item code and the first token of
  // the stage it holds (-1: past the end).
  take_ticket();
  uint4 kbuf[NBUF][SS], vbuf[NBUF][SS], qbuf[NBUF][HG];
  long slot_code[NBUF];
  int slot_t0[NBUF];
  ItemCursor cp = ld;
  long cp_code = ld_code;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) {
    load(kbuf[i], vbuf[i], qbuf[i], ld);
    slot_code[i] = ld_done ? -1 : ld_code;
    slot_t0[i] = ld.t0;
    ld_advance();
  }

  F st;
  st.set_q(qbuf[0], a.scale_log2);
  st.reset();
  for (;;) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      const int sl = (i + NBUF - 1) % NBUF;
      load(kbuf[sl], vbuf[sl], qbuf[sl], ld);
      slot_code[sl] = ld_done ? -1 : ld_code;
      slot_t0[sl] = ld.t0;
      ld_advance();
      __builtin_amdgcn_sched_barrier(0);
      st.fold(kbuf[i], vbuf[i], slot_t0[i], cp.end, r);
      if (slot_t0[i] + SUB >= cp.end) {
        const int h0 = (cp.y / a.head_chunks) * a.group + (cp.y % a.head_chunks) * HG;
        st.finish(a, (long)cp.b * a.num_q_heads + h0, num_parts(cp.L, P), cp.p, c, r);
        const int nx = (i + 1) % NBUF;
        const long next = slot_code[nx];
        if (next < 0) goto done;
        seek_item(cp, next, next == cp_code + 1, d, a, lens, lane);
        cp_code = next;
        st.set_q(qbuf[nx], a.scale_log2);
        st.reset();
      }
    }
  }
done:
  return;
}

// ---------------------------------------------------------------- combine

// One wave per (row, query head): rescale the partitions' partial outputs to
// a common max and normalise.  Lane p holds partition p's (max, sum); each
// lane owns D / 64 output elements.  The sums run over the partitions in
// order, so the result does not depend on which wave folded which partition.
// The row length, the first 64 partitions' (max, sum) pairs and the partial
// rows of partitions 0 and 1 (every row that needs a combine has both) are
// requested together; the partial rows of partitions 2 .. kPre - 1 follow
// once the length shows that the row has them.  So a two-partition row
// waits for one memory latency, and no partial row is read that the row
// does not have (indices stay inside the row's max_parts workspace entries).
constexpr int kCombinePre = 8;

template <typename E, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(RowAttnArgs a) {
  typedef typename E::storage T;
  constexpr int PER = D / 64;
  const long oh = blockIdx.x;
  const int row = (int)(oh / a.num_q_heads);
  const int lane = threadIdx.x;
  const float* ml = a.ws_ml + oh * a.max_parts * 2;
  const float* po = a.ws_o + oh * a.max_parts * D + lane * PER;
  const int Lraw = a.context_lens[row];
  float2 ml0 = make_float2(kNegBig, 0.f);
  if (lane < a.max_parts) ml0 = *reinterpret_cast<const float2*>(ml + 2 * lane);
  float pre[kCombinePre][PER];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[j][e] = po[(long)j * D + e];   // max_parts >= 2 here
  const int L = min(Lraw, a.max_context);
  const int nparts = num_parts(L, a.part_tokens);
  if (nparts <= 1) return;
#pragma unroll
  for (int j = 2; j < kCombinePre; ++j)
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[j][e] = j < nparts ? po[(long)j * D + e] : 0.f;
  float M = kNegBig;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    float mx = p0 + lane < nparts ? (p0 == 0 ? ml0.x : ml[2 * (p0 + lane)]) : kNegBig;
    mx = xor_max<32>(mx);
    mx = xor_max<16>(mx);
    mx = xor_max<8>(mx);
    mx = xor_max<4>(mx);
    mx = xor_max<2>(mx);
    mx = xor_max<1>(mx);
    M = fmaxf(M, mx);
  }
  float acc[PER], lsum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int n = min(64, nparts - p0);
    const bool in = lane < n;
    const float wl = in ? fast_exp2((p0 == 0 ? ml0.x : ml[2 * (p0 + lane)]) - M) : 0.f;
    const float ll = in ? (p0 == 0 ? ml0.y : ml[2 * (p0 + lane) + 1]) : 0.f;
    int j = 0;
    if (p0 == 0) {
#pragma unroll
      for (; j < kCombinePre; ++j) {
        if (j >= n) break;
        const float wg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
        lsum = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ll), j)), wg, lsum);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(pre[j][e], wg, acc[e]);
      }
    }
#pragma unroll 8
    for (; j < n; ++j) {
      const float wg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
      lsum = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ll), j)), wg, lsum);
      const float* pp = po + (long)(p0 + j) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(pp[e], wg, acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    E::store(reinterpret_cast<T*>(a.out) + oh * D + lane * PER + e, acc[e] / lsum);
}

// ---------------------------------------------------------------- launch

template <typename E, int D, int HG>
static int launch_persistent(const RowAttnArgs& a, hipStream_t stream) {
  // One wave per SIMD (never more than the kernel's occupancy allows).  Two
  // waves sharing a SIMD split its memory stream unevenly -- the older wave's
  // requests go first, and on the Qwen3 decode workload the younger one took
  // 2.6x as long over the same item, which left a long tail -- while one
  // wave per SIMD with two stages in flight already keeps HBM saturated.
  static std::atomic<int> slots_cache[kMaxDevices];
  static std::atomic<int> simds_cache[kMaxDevices];
  const int resident = resident_blocks(
      reinterpret_cast<const void*>(decode_persistent_kernel<E, D, HG>), 64, slots_cache);
  const int simds = device_simds(simds_cache);
  if (resident < 0 || simds < 0) return -1;
  const long long max_items =
      (long long)a.num_rows * a.num_kv_heads * a.head_chunks * a.max_parts;
  const int waves = (int)min((long long)min(resident, simds), max_items);
  if (waves <= 0) return 0;
  hipLaunchKernelGGL((decode_persistent_kernel<E, D, HG>), dim3(waves), dim3(64), 0, stream, a,
                     a.context_lens, a.block_tables);
  return 0;
}

template <typename E, int D, bool VARLEN, bool BIG>
static int launch_rows_hg(const RowAttnArgs& a, hipStream_t stream) {
  const long long grid =
      (long long)a.num_rows * a.num_kv_heads * a.head_chunks * a.max_parts;
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -1;
  const dim3 g((unsigned)grid), blk(64);
  switch (a.heads_per_wg) {
#define PA_HG_CASE(N)                                                                        \
  case N:                                                                                    \
    if constexpr (N <= (D == 64 ? 8 : 4)) {                                                  \
      if constexpr (BIG && !VARLEN)                                                          \
        return launch_persistent<E, D, N>(a, stream);                                        \
      else                                                                                   \
        hipLaunchKernelGGL((row_attn_kernel<E, D, N, VARLEN, BIG>), g, blk, 0, stream, a);   \
    } else {                                                                                 \
      return -1;                                                                             \
    }                                                                                        \
    break;
    PA_HG_CASE(1)
    PA_HG_CASE(2)
    PA_HG_CASE(3)
    PA_HG_CASE(4)
    PA_HG_CASE(5)
    PA_HG_CASE(6)
    PA_HG_CASE(7)
    PA_HG_CASE(8)
#undef PA_HG_CASE
    default:
      return -1;
  }
  return 0;
}

template <typename E, int D, bool VARLEN>
static int launch_rows_mode(const RowAttnArgs& a, hipStream_t stream) {
  if (a.block_size_log2 >= 6) return launch_rows_hg<E, D, VARLEN, true>(a, stream);
  return launch_rows_hg<E, D, VARLEN, false>(a, stream);
}

static int dispatch_rows(const RowAttnArgs& a, int head_dim, int dtype, bool varlen,
                         hipStream_t stream) {
  if (dtype == 0) {
    if (head_dim == 64)
      return varlen ? launch_rows_mode<ElemF32, 64, true>(a, stream)
                    : launch_rows_mode<ElemF32, 64, false>(a, stream);
    return varlen ? launch_rows_mode<ElemF32, 128, true>(a, stream)
                  : launch_rows_mode<ElemF32, 128, false>(a, stream);
  }
  if (varlen) return -1;  // bf16 prefill runs on the matrix cores
  return head_dim == 64 ? launch_rows_mode<ElemBF16, 64, false>(a, stream)
                        : launch_rows_mode<ElemBF16, 128, false>(a, stream);
}

int launch_decode(const RowAttnArgs& a, int head_dim, int dtype, hipStream_t stream) {
  // bf16 query groups of kGqaMfmaMinGroup heads or more fold on the matrix
  // cores (every block size, so results stay independent of it).
  const int mfma_heads = dtype == 1 ? gqa_mfma_heads(a.group, head_dim) : 0;
  int rc;
  if (mfma_heads > 0) {
    RowAttnArgs m = a;
    m.heads_per_wg = mfma_heads;
    m.head_chunks = a.group / mfma_heads;
    rc = launch_decode_gqa_mfma(m, head_dim, stream);
  } else {
    rc = dispatch_rows(a, head_dim, dtype, false, stream);
  }
  if (rc || a.max_parts <= 1) return rc;
  const dim3 g((unsigned)((long long)a.num_rows * a.num_q_heads));
  if (dtype == 0) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 64>), g, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 128>), g, dim3(64), 0, stream, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 64>), g, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 128>), g, dim3(64), 0, stream, a);
  }
  return 0;
}

int launch_varlen_rows(const RowAttnArgs& a, int head_dim, int dtype, hipStream_t stream) {
  return dispatch_rows(a, head_dim, dtype, true, stream);
}

}  // namespace pa
