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

template <typename E, int D, int HG, bool VARLEN>
__global__ __launch_bounds__(256) void row_attn_kernel(RowAttnArgs a) {
  typedef typename E::storage T;
  constexpr int EPL = E::EPL;
  constexpr int LPR = D / EPL;  // lanes per K/V head row
  constexpr int RPS = 64 / LPR;  // token rows per load instruction
  constexpr int S = 64 / RPS;    // load steps per 64-token chunk

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c = lane % LPR;
  const int r = lane / LPR;

  // blockIdx.x = (row * Y + y) * max_parts + p, Y = kv heads * head chunks
  const int Y = a.num_kv_heads * a.head_chunks;
  int x = blockIdx.x;
  const int p = x % a.max_parts;
  x /= a.max_parts;
  const int y = x % Y;
  const int row = x / Y;
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
      for (int idx = threadIdx.x; idx < HG * D; idx += 256)
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
  const bool big_blocks = bs_log2 >= 6;  // a 64-token chunk never straddles a block

  // Queries of the HG heads, pre-multiplied by scale * log2(e): scores come
  // out in log2 units and the softmax uses exp2.
  float qf[HG][EPL];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((long)row * a.num_q_heads + h0) * D + c * EPL;
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
  const long slot_elems = (long)a.num_kv_heads * D;
  const long head_off = (long)g * D + c * EPL;

  for (int t0 = tok_begin + w * 64; t0 < tok_end; t0 += 256) {
    long sbase = 0;
    if (big_blocks) {
      const int blk = clamp_block(bt[t0 >> bs_log2], nb);
      sbase = ((long)blk << bs_log2) - (long)((t0 >> bs_log2) << bs_log2);
    }
    uint4 kr[S], vr[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int j = t0 + s * RPS + r;
      if (j < tok_end) {
        long slot;
        if (big_blocks) {
          slot = sbase + j;
        } else if (bs_log2 >= 0) {
          slot = ((long)clamp_block(bt[j >> bs_log2], nb) << bs_log2) + (j & (bs - 1));
        } else {
          slot = (long)clamp_block(bt[j / bs], nb) * bs + j % bs;
        }
        const long off = slot * slot_elems + head_off;
        kr[s] = *reinterpret_cast<const uint4*>(kc + off);
        vr[s] = *reinterpret_cast<const uint4*>(vc + off);
      } else {
        kr[s] = make_uint4(0, 0, 0, 0);
        vr[s] = make_uint4(0, 0, 0, 0);
      }
    }

    float sc[HG][S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
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
    for (int s = 0; s < S; ++s) {
      const bool valid = t0 + s * RPS + r < tok_end;
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float v = group_sum<LPR>(sc[h][s]);
        sc[h][s] = valid ? v : -INFINITY;
      }
    }

#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float mx = sc[h][0];
#pragma unroll
      for (int s = 1; s < S; ++s) mx = fmaxf(mx, sc[h][s]);
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      float lsum = l[h] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const float pr = fast_exp2(sc[h][s] - mn);
        lsum += pr;
        sc[h][s] = pr;
      }
      l[h] = lsum;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float vf[EPL];
      E::widen(vr[s], vf);
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(sc[h][s], vf[e], o[h][e]);
    }
  }

  // Merge the RPS independent row states of the wave (lanes c, c + LPR, ...).
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

  // Merge the four waves through LDS and finish (or emit a partial).
  __shared__ float s_o[4][HG][D];
  __shared__ float s_ml[4][HG][2];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[w][h][c * EPL + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      s_ml[w][h][0] = m[h];
      s_ml[w][h][1] = l[h];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * D; idx += 256) {
    const int h = idx / D;
    const int d = idx % D;
    float M = s_ml[0][h][0];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, s_ml[ww][h][0]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float wg = fast_exp2(s_ml[ww][h][0] - M);
      acc = fmaf(s_o[ww][h][d], wg, acc);
      lsum = fmaf(s_ml[ww][h][1], wg, lsum);
    }
    const long oh = (long)row * a.num_q_heads + h0 + h;
    if (nparts == 1) {
      E::store(out + oh * D + d, acc / lsum);
    } else {
      a.ws_o[(oh * a.max_parts + p) * D + d] = acc;
      if (d == 0) {
        a.ws_ml[(oh * a.max_parts + p) * 2] = M;
        a.ws_ml[(oh * a.max_parts + p) * 2 + 1] = lsum;
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

template <typename E, int D, bool VARLEN>
static int launch_rows_hg(const RowAttnArgs& a, hipStream_t stream) {
  const long long grid =
      (long long)a.num_rows * a.num_kv_heads * a.head_chunks * a.max_parts;
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -1;
  const dim3 g((unsigned)grid), blk(256);
  switch (a.heads_per_wg) {
#define PA_HG_CASE(N)                                                                        \
  case N:                                                                                    \
    if constexpr (N <= (D == 64 ? 8 : 4))                                                    \
      hipLaunchKernelGGL((row_attn_kernel<E, D, N, VARLEN>), g, blk, 0, stream, a);          \
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

static int dispatch_rows(const RowAttnArgs& a, int head_dim, int dtype, bool varlen,
                         hipStream_t stream) {
  if (dtype == 0) {
    if (head_dim == 64)
      return varlen ? launch_rows_hg<ElemF32, 64, true>(a, stream)
                    : launch_rows_hg<ElemF32, 64, false>(a, stream);
    return varlen ? launch_rows_hg<ElemF32, 128, true>(a, stream)
                  : launch_rows_hg<ElemF32, 128, false>(a, stream);
  }
  if (varlen) return -1;  // bf16 prefill runs on the matrix cores
  return head_dim == 64 ? launch_rows_hg<ElemBF16, 64, false>(a, stream)
                        : launch_rows_hg<ElemBF16, 128, false>(a, stream);
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
