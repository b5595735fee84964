// Decode attention for large query groups on the gfx950 matrix cores.
//
// In a decode step each sequence brings one new query row per query head,
// and the heads of a KV head's group all read the same cached keys and
// values ("nano-vLLM Part 4", section 3: decode attention over the cached
// history through the block table).  When the group is large (Qwen2.5-0.5B:
// 14 query heads over 2 KV heads, a group of 7) the per-token work of the
// vector fold grows with the group, and a small batch -- whose time is one
// wave's context partition -- becomes bound by that wave's instruction
// stream.  The group's scores and outputs are dense contractions, so this
// kernel computes them with v_mfma_f32_16x16x32_bf16:
//
//     S^T (16 tokens x 16 heads)  = K (16 x D) . Q^T (D x 16)   (D / 32 MFMAs)
//     O^T (16 dims  x 16 heads)  += V^T (16 x 32) . P^T (32 x 16)  (per 16 dims)
//
// per 32-token chunk, with the group's heads (up to 16) in the 16 columns.
// Lane l owns head column l % 16; its four lane groups (l / 16) hold eight
// consecutive tokens of a chunk after the score products, because the K rows
// are fed to the two score MFMAs in a permuted order -- the probabilities
// then sit in exactly the layout of the output product's B operand, and go
// there without leaving the registers.  K rows load straight into the A
// operand (16 contiguous bytes of one token per lane); V passes through LDS,
// from which the transposed operand (8 tokens of one dimension per lane) is
// read with ds_read_b64_tr_b16.
//
// The unit of work, the partition size, the partial format and the combine
// are those of the vector kernels: an item is (sequence, 512-token
// partition, KV head [, chunk of 16 heads]), and a sequence with several
// partitions writes unnormalised partials that the combine kernel merges in
// partition order.  A workgroup of NW waves folds an item: wave w takes the
// w-th fixed quarter (part_tokens / NW tokens) of the partition, and the
// quarters' states are merged through LDS in wave order -- a fixed split, so
// a small batch gets NW times the waves without any change to a row's
// arithmetic.  A row's arithmetic depends only on its own tokens: results
// are bitwise independent of the batch, the physical block IDs and the block
// size (the block table is staged in LDS and every block size takes this
// kernel).
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8m __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4m __attribute__((ext_vector_type(4)));
typedef float f32x4m __attribute__((ext_vector_type(4)));
typedef unsigned u32x4m __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4m lds_bf16x4m;

namespace {

__device__ __forceinline__ float max_across_groups(float x) {
  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same head column
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_groups(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (unsigned)__builtin_bit_cast(uint16_t, a) | ((unsigned)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace

// D: head dim (64 or 128); NST: register stages in the ring; NW: waves per
// item.
template <int D, int NST, int NW>
__global__ __launch_bounds__(64 * NW) void decode_gqa_mfma_kernel(RowAttnArgs a) {
  constexpr int KC = D / 32;            // 32-dim chunks of the score products
  constexpr int NBD = D / 16;           // 16-dim blocks of the output products
  constexpr int CPR = D / 8;            // 16-byte chunks per head row
  constexpr int VL = 32 * CPR / 64;     // V loads per lane per 32-token chunk
  constexpr int RS = D + (D == 64 ? 8 : 16);  // LDS row stride (elements), padded for the transpose reads
  constexpr int CH = 32;                // tokens per chunk

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;      // wave of the item
  const int col = lane & 15;            // head column
  const int grp = lane >> 4;            // lane group: k rows 8*grp .. 8*grp + 7

  // blockIdx.x = (row * max_parts + p) * Y + y, Y = kv heads * head chunks
  const int Y = a.num_kv_heads * a.head_chunks;
  const int HG = a.heads_per_wg;
  int x = blockIdx.x;
  const int y = x % Y;
  x /= Y;
  const int p = x % a.max_parts;
  const int row = x / a.max_parts;
  const int g = y / a.head_chunks;
  const int h0 = g * a.group + (y % a.head_chunks) * HG;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const int32_t* bt = a.block_tables + (long)row * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nb = a.num_blocks;
  const int part_begin = p * a.part_tokens;
  const int first_blk = bs_log2 >= 0 ? (part_begin >> bs_log2) : part_begin / bs;

  // The block IDs of the partition's whole span (within the table's width)
  // and the query are loaded together with the sequence length, so that one
  // memory round trip, not three, precedes the key/value loads.  Entries
  // past the sequence's end are staged too (clamped) and never used.
  constexpr int BPT = (kDecodePartition + 64 * NW - 1) / (64 * NW);
  int btv[BPT];
  {
    const int span_end = part_begin + a.part_tokens - 1;
    const int last_span = bs_log2 >= 0 ? (span_end >> bs_log2) : span_end / bs;
    const int nspan = min(min(last_span, a.max_blocks_per_seq - 1) - first_blk + 1, kDecodePartition);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int i = (int)threadIdx.x + k * 64 * NW;
      btv[k] = i < nspan ? bt[first_blk + i] : -1;
    }
  }

  // Query operand (B of the score products): head column `col`, dims
  // 32 * kc + 8 * grp .. + 7.  Columns past the group hold zeros.
  bf16x8m qB[KC];
  {
    const bool live = col < HG;
    const u32x4m* qp = reinterpret_cast<const u32x4m*>(
        reinterpret_cast<const uint16_t*>(a.q) + ((long)row * a.num_q_heads + h0 + (live ? col : 0)) * D +
        8 * grp);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const u32x4m v = live ? qp[4 * kc] : u32x4m{0u, 0u, 0u, 0u};
      qB[kc] = __builtin_bit_cast(bf16x8m, v);
    }
  }

  const int L = min(a.context_lens[row], a.max_context);
  if (L <= 0) {  // violated precondition: define the output as zeros
    if (p == 0)
      for (int idx = threadIdx.x; idx < HG * D; idx += 64 * NW)
        out[((long)row * a.num_q_heads + h0) * D + idx] = 0;
    return;
  }
  const int nparts = num_parts(L, a.part_tokens);
  if (p >= nparts) return;
  const int part_end = min(L, part_begin + a.part_tokens);
  // This wave's quarter of the partition (possibly empty).
  const int quarter = a.part_tokens / NW;
  const int tok_begin = part_begin + wv * quarter;
  const int tok_end = min(part_end, tok_begin + quarter);

  // The partition's block IDs, clamped into the pool; each wave's V staging
  // rows; the quarters' states for the merge.
  __shared__ int s_bt[kDecodePartition];
  __shared__ __attribute__((aligned(16))) uint16_t s_vall[NW][CH * RS];
  __shared__ float s_state[NW - 1][D / 4 + 2][64];
  uint16_t* s_v = s_vall[wv];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int i = (int)threadIdx.x + k * 64 * NW;
    if (i < kDecodePartition) s_bt[i] = clamp_block(btv[k], nb);
  }
  __syncthreads();

  const uint16_t* kcache = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vcache = reinterpret_cast<const uint16_t*>(a.v_cache);
  const long slot_elems = (long)a.num_kv_heads * D;
  const long head_off = (long)g * D;

  // Element offset of token t's row of this KV head (t is clamped to the
  // last valid token, so rows past the end repeat a written row).
  auto row_off = [&](int t) __attribute__((always_inline)) {
    t = min(t, tok_end - 1);
    int blk, in_blk;
    if (bs_log2 >= 0) {
      blk = t >> bs_log2;
      in_blk = t & (bs - 1);
    } else {
      blk = t / bs;
      in_blk = t - blk * bs;
    }
    return ((long)s_bt[blk - first_blk] * bs + in_blk) * slot_elems + head_off;
  };

  // One chunk of 32 tokens starting at c0: the K operand rows (half hf, row
  // i = col feeds token 8 * (i / 4) + 4 * hf + i % 4) and the V rows (load
  // j: token (64 * j + lane) / CPR, 16-byte chunk lane % CPR).
  auto load = [&](u32x4m (&kr)[2][KC], u32x4m (&vr)[VL], int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const long o = row_off(c0 + 8 * (col >> 2) + 4 * hf + (col & 3)) + 8 * grp;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kr[hf][kc] = *reinterpret_cast<const u32x4m*>(kcache + o + 32 * kc);
    }
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int s = 64 * j + lane;
      const long o = row_off(c0 + s / CPR) + 8 * (s % CPR);
      vr[j] = *reinterpret_cast<const u32x4m*>(vcache + o);
    }
  };

  f32x4m oacc[NBD];
#pragma unroll
  for (int n = 0; n < NBD; ++n) oacc[n] = f32x4m{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig;  // running max of the scaled scores (log2 units)
  float l_lane = 0.f;     // this lane's share of the running sum
  const float scale_log2 = a.scale_log2;

  auto fold = [&](const u32x4m (&kr)[2][KC], const u32x4m (&vr)[VL], int c0) __attribute__((always_inline)) {
    // Stage V (row-major, padded rows) for the transposed reads.
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int s = 64 * j + lane;
      *reinterpret_cast<u32x4m*>(s_v + (s / CPR) * RS + 8 * (s % CPR)) = vr[j];
    }
    // Scores: lane (col, grp) receives tokens c0 + 8 * grp + 4 * hf + e.
    f32x4m sc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sc[hf] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        sc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8m, kr[hf][kc]),
                                                         qB[kc], sc[hf], 0, 0, 0);
    }
    float s8[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = c0 + 8 * grp + 4 * hf + e;
        s8[4 * hf + e] = t < tok_end ? sc[hf][e] * scale_log2 : -INFINITY;
      }
    float mx = s8[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s8[e]);
    mx = max_across_groups(mx);
    const float mn = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - mn);
    m_run = mn;
    float pr[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(s8[e] - mn);
      ps += pr[e];
    }
    l_lane = fmaf(l_lane, alpha, ps);
    const u32x4m pw = {pack2(pr[0], pr[1]), pack2(pr[2], pr[3]), pack2(pr[4], pr[5]),
                       pack2(pr[6], pr[7])};
    const bf16x8m pB = __builtin_bit_cast(bf16x8m, pw);
    // Output products: A = V^T (16 dims x 32 tokens) from LDS, transposed.
    // Within a 16-lane group, lane m points at row 8 * grp + m / 4 (+ 4),
    // dims 16 * n + 4 * (m % 4): lane i then receives dim 16 * n + i of
    // rows 8 * grp .. + 3 (first read) and + 4 .. + 7 (second).
    const uint16_t* vb = s_v + (8 * grp + (col >> 2)) * RS + 4 * (col & 3);
#pragma unroll
    for (int n = 0; n < NBD; ++n) {
      const bf16x4m lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4m*)(vb + 16 * n));
      const bf16x4m hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4m*)(vb + 4 * RS + 16 * n));
      const bf16x8m vA = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[n][e] *= alpha;
      oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pB, oacc[n], 0, 0, 0);
    }
  };

  // Ring of NST register stages (NST - 1 chunks in flight while one is
  // folded); past the last chunk the loads repeat the last chunk.
  if (tok_begin < tok_end) {
    u32x4m kbuf[NST][2][KC], vbuf[NST][VL];
    const int last_c0 = tok_begin + ((tok_end - tok_begin - 1) / CH) * CH;
    int c0 = tok_begin;
#pragma unroll
    for (int i = 0; i < NST - 1; ++i) load(kbuf[i], vbuf[i], min(c0 + i * CH, last_c0));
    for (;;) {
#pragma unroll
      for (int i = 0; i < NST; ++i) {
        load(kbuf[(i + NST - 1) % NST], vbuf[(i + NST - 1) % NST],
             min(c0 + (NST - 1) * CH, last_c0));
        __builtin_amdgcn_sched_barrier(0);
        fold(kbuf[i], vbuf[i], c0);
        if (c0 >= last_c0) goto folded;
        c0 += CH;
      }
    }
  }
folded:
  // Merge the quarters in wave order: M = max of the quarters' maxima, then
  // O and the lane sums rescaled to M and summed wave 0 first.  (An empty
  // quarter has max kNegBig and weight 0.)
  if (wv > 0) {
#pragma unroll
    for (int n = 0; n < NBD; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_state[wv - 1][4 * n + e][lane] = oacc[n][e];
    s_state[wv - 1][D / 4][lane] = m_run;
    s_state[wv - 1][D / 4 + 1][lane] = l_lane;
  }
  __syncthreads();
  if (wv > 0) return;
  {
    float M = m_run;
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_state[w - 1][D / 4][lane]);
    const float w0 = fast_exp2(m_run - M);
#pragma unroll
    for (int n = 0; n < NBD; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[n][e] *= w0;
    l_lane *= w0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float ww = fast_exp2(s_state[w - 1][D / 4][lane] - M);
#pragma unroll
      for (int n = 0; n < NBD; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[n][e] = fmaf(s_state[w - 1][4 * n + e][lane], ww, oacc[n][e]);
      l_lane = fmaf(s_state[w - 1][D / 4 + 1][lane], ww, l_lane);
    }
    m_run = M;
  }
  // Output: lane (col, grp) holds head col's dims 16 * n + 4 * grp + e.
  {
    const float l_tot = sum_across_groups(l_lane);
    if (col >= HG) return;
    const long oh = (long)row * a.num_q_heads + h0 + col;
    if (nparts == 1) {
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int n = 0; n < NBD; ++n) {
        const uint2 w = make_uint2(pack2(oacc[n][0] * inv, oacc[n][1] * inv),
                                   pack2(oacc[n][2] * inv, oacc[n][3] * inv));
        *reinterpret_cast<uint2*>(out + oh * D + 16 * n + 4 * grp) = w;
      }
    } else {
      float* po = a.ws_o + (oh * a.max_parts + p) * D + 4 * grp;
#pragma unroll
      for (int n = 0; n < NBD; ++n)
        *reinterpret_cast<float4*>(po + 16 * n) =
            make_float4(oacc[n][0], oacc[n][1], oacc[n][2], oacc[n][3]);
      if (grp == 0) {
        a.ws_ml[(oh * a.max_parts + p) * 2] = m_run;
        a.ws_ml[(oh * a.max_parts + p) * 2 + 1] = l_tot;
      }
    }
  }
}

// Heads per item for the matrix path: the whole group when it fits the 16
// columns, else 16 when the group is a multiple of 16; 0 when the group is
// not served here.
int gqa_mfma_heads(int group, int head_dim) {
  if (head_dim != 64 && head_dim != 128) return 0;
  if (group >= kGqaMfmaMinGroup && group <= 16) return group;
  if (group > 16 && group % 16 == 0) return 16;
  return 0;
}

#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 4
#endif
constexpr int kGqaWaves = PA_GQA_WAVES;  // waves (fixed token quarters) per item
#ifndef PA_GQA_STAGES_D64
#define PA_GQA_STAGES_D64 3
#endif
#ifndef PA_GQA_STAGES_D128
#define PA_GQA_STAGES_D128 3
#endif

int launch_decode_gqa_mfma(const RowAttnArgs& a, int head_dim, hipStream_t stream) {
  const long long grid =
      (long long)a.num_rows * a.num_kv_heads * a.head_chunks * a.max_parts;
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -1;
  static_assert(kDecodePartition % (32 * kGqaWaves) == 0, "partition quarters hold whole chunks");
  if (head_dim == 64)
    hipLaunchKernelGGL((decode_gqa_mfma_kernel<64, PA_GQA_STAGES_D64, kGqaWaves>),
                       dim3((unsigned)grid), dim3(64 * kGqaWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_gqa_mfma_kernel<128, PA_GQA_STAGES_D128, kGqaWaves>),
                       dim3((unsigned)grid), dim3(64 * kGqaWaves), 0, stream, a);
  return 0;
}

}  // namespace pa
