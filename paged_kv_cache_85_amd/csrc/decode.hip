// Decode attention over a paged KV cache on the vector ALUs, split over the
// context ("flash-decoding" style partitions) with an online softmax.
//
// A decode query is one token per sequence attending to that sequence's
// cached keys and values ("mini-vLLM", project summary), read through the
// sequence's block table ("nano-vLLM Part 4", section 3: decode attention
// over the cached history).  The work is HBM-bound (about 2 FLOP per byte of
// bf16 KV at a query group of 2), so the kernel is organised around the
// memory stream rather than the matrix cores:
//
//  * one workgroup = 4 waves = one (sequence, KV head, context partition);
//    the query heads of the KV head's group (up to HG of them) share every
//    K/V row loaded, so each KV byte is read once per group;
//  * a wave covers 64 tokens per iteration; each lane loads 16 contiguous
//    bytes of a token's head row, LPR lanes cover the row and RPS rows load
//    per instruction, so every load is a fully used 16-byte access and a wave
//    keeps 2 x 64 x 16 B x (64 / RPS) bytes in flight;
//  * q.k partial dot products are reduced across the LPR lanes of a row with
//    DPP (quad permutes and row mirrors), which leaves every lane of the row
//    holding the full score, so probabilities need no broadcast;
//  * each lane row keeps its own running max / sum / output (an independent
//    online softmax), merged across rows and waves once at the end;
//  * partitions of several 64-token chunks write unnormalised partials
//    (output, max, sum) to the workspace; a small combine kernel rescales and
//    sums them.  A sequence that fits one partition is finished in place.
//
// The same kernel, in "varlen" mode, computes fp32 prefill rows: row i of a
// sequence with Lq new and Lk total tokens is a decode over its first
// Lk - Lq + i + 1 keys.
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

// BIG: power-of-two blocks of >= 64 tokens, so a pipeline stage never
// straddles a block and one scalar table read serves a stage.  Otherwise
// decode stages its partition's block IDs in LDS (one read at the start, so
// lookups never wait behind the K/V stream) and varlen rows read the table
// per lane.
template <typename E, int D, int HG, bool VARLEN, bool BIG>
__global__ __launch_bounds__(64) void row_attn_kernel(RowAttnArgs a) {
  typedef typename E::storage T;
  constexpr int EPL = E::EPL;
  constexpr int LPR = D / EPL;   // lanes per K/V head row
  constexpr int RPS = 64 / LPR;  // token rows per load instruction
  constexpr int SS = 8;          // load steps per pipeline stage
  constexpr int SUB = SS * RPS;  // tokens per pipeline stage (16..64)

  const int lane = threadIdx.x;
  const int c = lane % LPR;
  const int r = lane / LPR;

  // blockIdx.x = (row * max_parts + p) * Y + y, Y = kv heads * head chunks:
  // the heads of one partition are adjacent, so they are dispatched together
  // and read neighbouring bytes of the same token rows.
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

  T* out = reinterpret_cast<T*>(a.out);
  if (L <= 0) {  // violated precondition: define the output as zeros
    if (p == 0)
      for (int idx = lane; idx < HG * D; idx += 64)
        E::store(out + ((long)row * a.num_q_heads + h0) * D + idx, 0.f);
    return;
  }
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (p >= nparts) return;
  const int tok_begin = p * a.part_tokens;
  const int tok_end = min(L, tok_begin + a.part_tokens);
  const int32_t* bt = a.block_tables + (long)b * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nb = a.num_blocks;

  constexpr bool kLdsTable = !BIG && !VARLEN;
  constexpr int kMaxTable = kLdsTable ? 256 : 1;  // blocks of one 256-token partition
  __shared__ int s_bt[kMaxTable];
  int first_blk = 0;
  if constexpr (kLdsTable) {
    first_blk = bs_log2 >= 0 ? (tok_begin >> bs_log2) : tok_begin / bs;
    const int last_blk = bs_log2 >= 0 ? ((tok_end - 1) >> bs_log2) : (tok_end - 1) / bs;
    for (int i = lane; i <= last_blk - first_blk && i < kMaxTable; i += 64)
      s_bt[i] = clamp_block(bt[first_blk + i], nb);
    __syncthreads();
  }

  // Queries of the HG heads, pre-multiplied by scale * log2(e): scores come
  // out in log2 units and the softmax uses exp2.
  float qf[HG][EPL];
  {
    const T* qp =
        reinterpret_cast<const T*>(a.q) + ((long)row * a.num_q_heads + h0) * D + c * EPL;
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      E::widen(*reinterpret_cast<const uint4*>(qp + h * D), qf[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] *= a.scale_log2;
    }
  }

  float m[HG], l[HG], o[HG][EPL];
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  const T* kc = reinterpret_cast<const T*>(a.k_cache);
  const T* vc = reinterpret_cast<const T*>(a.v_cache);
  const int slot_elems = a.num_kv_heads * D;  // elements per token slot
  const int head_off = g * D + c * EPL;
  unsigned big_off[BIG ? SS : 1];
  if constexpr (BIG) {
#pragma unroll
    for (int s = 0; s < SS; ++s)
      big_off[s] = (unsigned)((s * RPS + r) * slot_elems + c * EPL) * (unsigned)sizeof(T);
  }

  // Load one stage of SUB tokens.  Lanes past the partition's end read the
  // last valid token instead (always a written row, never poison) and their
  // scores are masked, so every load is unconditional and in bounds.
  auto load = [&](uint4 (&kr)[SS], uint4 (&vr)[SS], int t0) {
    const int nvalid = tok_end - t0;  // >= 1
    if constexpr (BIG) {
      // Wave-uniform base of this stage's rows for head g plus loop-invariant
      // per-lane byte offsets.  A stage lies inside one block, so rows past
      // the partition's end are still pool slots of that block (possibly
      // poison); compute() masks their scores and zeroes their values.
      const int blk = clamp_block(bt[t0 >> bs_log2], nb);
      const long base = (((long)blk << bs_log2) + (t0 & (bs - 1))) * slot_elems + (long)g * D;
      const char* kp = reinterpret_cast<const char*>(kc + base);
      const char* vp = reinterpret_cast<const char*>(vc + base);
#pragma unroll
      for (int s = 0; s < SS; ++s) kr[s] = *reinterpret_cast<const uint4*>(kp + big_off[s]);
#pragma unroll
      for (int s = 0; s < SS; ++s) vr[s] = *reinterpret_cast<const uint4*>(vp + big_off[s]);
    } else {
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
      for (int s = 0; s < SS; ++s) kr[s] = *reinterpret_cast<const uint4*>(kc + off[s]);
#pragma unroll
      for (int s = 0; s < SS; ++s) vr[s] = *reinterpret_cast<const uint4*>(vc + off[s]);
    }
  };

  // Fold one stage into the running (max, sum, output) of this lane's row.
  auto compute = [&](const uint4 (&kr)[SS], const uint4 (&vr)[SS], int t0) {
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
    uint4 vz[SS];
#pragma unroll
    for (int s = 0; s < SS; ++s) vz[s] = vr[s];
    if (t0 + SUB > tok_end) {  // last, partial stage: rows past the end do not count
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const bool valid = t0 + s * RPS + r < tok_end;
#pragma unroll
        for (int h = 0; h < HG; ++h) sc[h][s] = valid ? sc[h][s] : -INFINITY;
        if (!valid) vz[s] = make_uint4(0, 0, 0, 0);
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
      E::widen(vz[s], vf);
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(sc[h][s], vf[e], o[h][e]);
    }
  };

  // Two register stages: the next stage's loads are in flight while the
  // current one is folded in.  The prefetch is unconditional (at the end it
  // re-reads the last stage, which is cached) so that the compiler can count
  // outstanding loads exactly and never waits for the stage in flight.
  uint4 kA[SS], vA[SS], kB[SS], vB[SS];
  const int last_t0 = tok_begin + ((tok_end - tok_begin - 1) / SUB) * SUB;
  int t0 = tok_begin;
  load(kA, vA, t0);
  // sched_barrier keeps the scheduler from sinking the prefetch below the
  // fold of the current stage.
  for (;;) {
    load(kB, vB, min(t0 + SUB, last_t0));
    __builtin_amdgcn_sched_barrier(0);
    compute(kA, vA, t0);
    if (t0 >= last_t0) break;
    t0 += SUB;
    load(kA, vA, min(t0 + SUB, last_t0));
    __builtin_amdgcn_sched_barrier(0);
    compute(kB, vB, t0);
    if (t0 >= last_t0) break;
    t0 += SUB;
  }

  // Merge the RPS independent row states (lanes c, c + LPR, ...).
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float M = m[h];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float wgt = fast_exp2(m[h] - M);
    float lw = l[h] * wgt;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float ov = o[h][e] * wgt;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) ov += __shfl_xor(ov, off);
      o[h][e] = ov;
    }
    m[h] = M;
    l[h] = lw;
  }

  if (r != 0) return;
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const long oh = (long)row * a.num_q_heads + h0 + h;
    if (nparts == 1) {
      const float inv = 1.f / l[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) E::store(out + oh * D + c * EPL + e, o[h][e] * inv);
    } else {
      float* po = a.ws_o + (oh * a.max_parts + p) * D + c * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(po + e) = make_float4(o[h][e], o[h][e + 1], o[h][e + 2],
                                                         o[h][e + 3]);
      if (c == 0) {
        a.ws_ml[(oh * a.max_parts + p) * 2] = m[h];
        a.ws_ml[(oh * a.max_parts + p) * 2 + 1] = l[h];
      }
    }
  }
}

// One block of D threads per (row, query head): rescale the partitions'
// partial outputs to a common max and normalise.
template <typename E, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(RowAttnArgs a) {
  typedef typename E::storage T;
  const long oh = blockIdx.x;
  const int row = (int)(oh / a.num_q_heads);
  const int L = min(a.context_lens[row], a.max_context);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const float* ml = a.ws_ml + oh * a.max_parts * 2;
  float M = kNegBig;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  const float* po = a.ws_o + oh * a.max_parts * D + threadIdx.x;
  float acc = 0.f, lsum = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float wg = fast_exp2(ml[2 * p] - M);
    acc = fmaf(po[(long)p * D], wg, acc);
    lsum = fmaf(ml[2 * p + 1], wg, lsum);
  }
  E::store(reinterpret_cast<T*>(a.out) + oh * D + threadIdx.x, acc / lsum);
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
    if constexpr (N <= (D == 64 ? 8 : 4))                                                    \
      hipLaunchKernelGGL((row_attn_kernel<E, D, N, VARLEN, BIG>), g, blk, 0, stream, a);     \
    else                                                                                     \
      return -1;                                                                             \
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
  int rc = dispatch_rows(a, head_dim, dtype, false, stream);
  if (rc || a.max_parts <= 1) return rc;
  const dim3 g((unsigned)((long long)a.num_rows * a.num_q_heads));
  if (dtype == 0) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 64>), g, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_combine_kernel<ElemF32, 128>), g, dim3(128), 0, stream, a);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 64>), g, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_combine_kernel<ElemBF16, 128>), g, dim3(128), 0, stream, a);
  }
  return 0;
}

int launch_varlen_rows(const RowAttnArgs& a, int head_dim, int dtype, hipStream_t stream) {
  return dispatch_rows(a, head_dim, dtype, true, stream);
}

}  // namespace pa
