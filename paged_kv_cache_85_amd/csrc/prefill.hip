// Varlen causal prefill over a paged KV cache on the gfx950 matrix cores
// (bf16 inputs, fp32 accumulation).
//
// Packed prompts attend causally to themselves ("mini-vLLM", project
// summary); sequence boundaries come from cu_seqlens_q / cu_seqlens_k, and
// cu_seqlens_k > cu_seqlens_q means the sequence already has a cached prefix
// (smzdm Nano-vLLM walk-through, model implementation details), so its Lq new
// rows are the last rows of the sequence: row i sees keys 0 .. Lk - Lq + i.
// All keys are read from the pools through the block table.
//
// Tiling.  A workgroup (4 waves) owns one KV head, HPW of its query heads and
// BMQ = 32 * (4 / HPW) consecutive query rows; each wave owns 32 rows of one
// head.  Key/value tiles of 64 tokens are gathered through the block table
// into LDS once per workgroup (double-buffered) and shared by all four waves.
// Per tile a wave computes
//     S^T (64 keys x 32 rows)  = K_tile . Q^T       (v_mfma_f32_32x32x16_bf16)
//     O^T (D x 32 rows)       += V_tile^T . P^T
// Computing the transposed products puts each query row in one lane (and its
// mirror lane 32 apart), so the row max / row sum of the online softmax are
// in-lane reductions plus one exchange.  K rows are fed to the first MFMA in
// a permuted order (bits 2 and 3 of the row index swapped) so that the fp32
// scores a lane receives are exactly the 8-consecutive-key runs that the
// second MFMA expects as its B operand: P goes from the score registers to
// the PV product without touching LDS.  V stays row-major in LDS; its
// transposed operand (8 consecutive keys of one head-dim column per lane) is
// read with the gfx950 LDS transpose load (ds_read_b64_tr_b16), two per
// operand.
//
// LDS layouts (row strides chosen for conflict-free access):
//   K: row stride D + 8 elements -- consecutive rows shift by 16 bytes, so
//      the 16 lanes of an operand read (16 different rows, same column) hit
//      16 different 16-byte bank groups;
//   V: row stride D + 32 elements -- consecutive rows shift by a quarter of
//      the 256-byte bank space, so the 4 keys x 64 bytes of a transpose read
//      cover all banks once.
//
// Work order: the grid runs the last (heaviest, under the causal mask) query
// tiles of every sequence first.  Tiles entirely above the diagonal are
// skipped; masking is applied only to tiles that cross it.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int swap_bits_2_3(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t prefill_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// LDS transpose read: within each 16-lane group, lane j points at 4
// consecutive 16-bit elements (chunk j); lane i receives element
// chunk[4k + i/4][i%4] as its k-th value.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

template <int D, int HPW, bool BIG>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BN = 64;             // keys per tile
  constexpr int WPH = 4 / HPW;       // waves per query head
  constexpr int BMQ = 32 * WPH;      // query rows per workgroup
  constexpr int KC = D / 16;         // k-steps of the QK^T product
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int KS = D + 8;          // LDS row stride of K (elements)
  constexpr int VS = D + 32;         // LDS row stride of V (elements)
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int CPT = BN * CPR / 256;  // chunks per thread per tile
  constexpr int RPI = 256 / CPR;     // tile rows covered per chunk index i

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  const int hchunks = a.group / HPW;
  const int inner = a.num_kv_heads * hchunks;
  int x = blockIdx.x;
  const int gh = x % inner;
  x /= inner;
  const int b = x % a.num_seqs;
  const int qt_rev = x / a.num_seqs;
  const int n_qt = (a.max_seqlen_q + BMQ - 1) / BMQ;
  const int qt = n_qt - 1 - qt_rev;
  const int g = gh / hchunks;
  const int hc = gh % hchunks;

  const int q_start = a.cu_seqlens_q[b];
  if (q_start < 0 || q_start >= a.total_q) return;
  const int Lk = min(min(a.cu_seqlens_k[b + 1] - a.cu_seqlens_k[b], a.max_seqlen_k),
                     a.max_blocks_per_seq * a.block_size);
  const int Lq = min(min(min(a.cu_seqlens_q[b + 1] - q_start, a.max_seqlen_q), Lk),
                     a.total_q - q_start);
  if (qt < 0 || qt * BMQ >= Lq) return;
  const int delta = Lk - Lq;

  const int head_local = w / WPH;
  const int h = g * a.group + hc * HPW + head_local;
  const int row0 = qt * BMQ + (w % WPH) * 32;  // first row of this wave in the sequence
  const bool wave_active = row0 < Lq;
  const int kmax_wave = delta + min(row0 + 32, Lq) - 1;
  const int kmax_wg = delta + min(qt * BMQ + BMQ, Lq) - 1;
  const int n_tiles = kmax_wg / BN + 1;

  // Q rows of this wave: B operand of S^T = K Q^T (lane holds 8 consecutive
  // head-dim elements of row lr for each 16-wide k-step).
  bf16x8 qB[KC];
  {
    const int qrow = row0 + lr;
    if (wave_active && qrow < Lq) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           ((long)(q_start + qrow) * a.num_q_heads + h) * D + lh * 8;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qB[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
    } else {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qB[kk] = bf16x8{};
    }
  }

  const uint16_t* kcache = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vcache = reinterpret_cast<const uint16_t*>(a.v_cache);
  const int32_t* bt = a.block_tables + (long)b * a.max_blocks_per_seq;
  const int slot_elems = a.num_kv_heads * D;
  const unsigned row_bytes = (unsigned)slot_elems * 2u;
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nblk = a.num_blocks;

  // Tile chunk i of this thread: row tid / CPR + RPI * i, 16-byte column tid % CPR.
  const int trow = tid / CPR;
  const int tcol = tid % CPR;
  unsigned big_off[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    big_off[i] = (unsigned)(trow + RPI * i) * row_bytes + (unsigned)(tcol * 16);

  uint4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int kt) {
    const int t0 = kt * BN;
    if constexpr (BIG) {
      // The 64-key tile lies in one block; rows past Lk fall outside the
      // descriptor and read zero.
      const int blk = clamp_block(bt[t0 >> bs_log2], nblk);
      const long base = (((long)blk << bs_log2) + (t0 & (bs - 1))) * slot_elems + (long)g * D;
      const unsigned bytes = (unsigned)min(BN, Lk - t0) * row_bytes;
      const __amdgpu_buffer_rsrc_t rk = prefill_rsrc(kcache + base, bytes);
      const __amdgpu_buffer_rsrc_t rv = prefill_rsrc(vcache + base, bytes);
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, big_off[i], 0, 0));
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        vreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, big_off[i], 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int j = t0 + trow + RPI * i;
        if (j < Lk) {
          long slot;
          if (bs_log2 >= 0)
            slot = ((long)clamp_block(bt[j >> bs_log2], nblk) << bs_log2) + (j & (bs - 1));
          else
            slot = (long)clamp_block(bt[j / bs], nblk) * bs + j % bs;
          const long off = slot * slot_elems + (long)g * D + tcol * 8;
          kreg[i] = *reinterpret_cast<const uint4*>(kcache + off);
          vreg[i] = *reinterpret_cast<const uint4*>(vcache + off);
        } else {
          kreg[i] = make_uint4(0, 0, 0, 0);
          vreg[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int row = trow + RPI * i;
      *reinterpret_cast<uint4*>(&sK[buf][row * KS + tcol * 8]) = kreg[i];
      *reinterpret_cast<uint4*>(&sV[buf][row * VS + tcol * 8]) = vreg[i];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.f;
  const int my_row = row0 + lr;
  const int klim = delta + my_row;  // last key this lane's row may see
  const int krow_perm = swap_bits_2_3(lr);
  // Transpose-read address pieces: 16-lane group q = lane / 16 covers head-dim
  // columns 16 * (q % 2) .. + 15 of keys 8 * (q / 2) + 4 * half + 0..3.
  const int tr_j = lane & 15;
  const int tr_key = 8 * lh + tr_j / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);

  load_tile(0);
  store_tile(0);
  if (n_tiles > 1) load_tile(1);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (wave_active && kt * BN <= kmax_wave) {
      f32x16 sacc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        sacc[nb] = f32x16{};
        const uint16_t* kp = &sK[buf][(nb * 32 + krow_perm) * KS + lh * 8];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(kp + kk * 16);
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qB[kk], sacc[nb], 0, 0, 0);
        }
      }
      // Lane (row lr, half lh) holds, in item t of block nb, the raw score of
      // key kt*64 + nb*32 + 16*(t/8) + 8*lh + t%8.
      const bool need_mask = (kt * BN + BN - 1 > delta + row0) || (kt * BN + BN > Lk);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int key = kt * BN + nb * 32 + 16 * (t >> 3) + 8 * lh + (t & 7);
            if (key > klim || key >= Lk) sacc[nb][t] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < 16; ++t) mx = fmaxf(mx, sacc[nb][t]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;  // scale > 0: max commutes with it
      // Lazy rescale: the reference max m_run only moves when a row's max
      // exceeds it by more than 2^8 (so probabilities stay <= 256); the final
      // O / l is the same for any reference, and the 64 multiplies of the O
      // rescale are skipped for every tile that does not move it.
      if (__any(mx > m_run + 8.f)) {
        const float mn = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int t = 0; t < 16; ++t) oacc[db][t] *= alpha;
      }
      float psum = 0.f;
      bf16x8 pB[4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pr = fast_exp2(fmaf(sacc[nb][half * 8 + e], a.scale_log2, -m_run));
            psum += pr;
            pB[nb * 2 + half][e] = (__bf16)pr;
          }
        }
      }
      l_run += psum;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* vp = &sV[buf][(kc * 16 + tr_key) * VS + db * 32 + tr_col];
          const bf16x4 lo = lds_read_tr(vp);
          const bf16x4 hi = lds_read_tr(vp + 4 * VS);
          const bf16x8 A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, pB[kc], oacc[db], 0, 0, 0);
        }
      }
    }
    // Stage the prefetched tile into the other buffer, then fetch the next.
    if (kt + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (kt + 2 < n_tiles) load_tile(kt + 2);
    }
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_row < Lq) {
    const float inv = 1.f / l_tot;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                   ((long)(q_start + my_row) * a.num_q_heads + h) * D;
    // Item t of block db is head-dim element db*32 + 8*(t/4) + 4*lh + t%4.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        uint2 u;
        u.x = pack_bf16x2(oacc[db][t4 * 4 + 0] * inv, oacc[db][t4 * 4 + 1] * inv);
        u.y = pack_bf16x2(oacc[db][t4 * 4 + 2] * inv, oacc[db][t4 * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * t4 + 4 * lh) = u;
      }
    }
  }
}

template <int D, int HPW>
static int launch_hpw(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BMQ = 32 * (4 / HPW);
  const long long n_qt = (a.max_seqlen_q + BMQ - 1) / BMQ;
  const long long grid =
      n_qt * a.num_seqs * (long long)a.num_kv_heads * (a.group / HPW);
  if (grid <= 0) return 0;
  if (grid > 0x7fffffffLL) return -1;
  if (a.block_size_log2 >= 6)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, HPW, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, HPW, false>), dim3((unsigned)grid), dim3(256), 0,
                       stream, a);
  return 0;
}

int launch_prefill_bf16(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  const int hpw = (a.group % 4 == 0) ? 4 : (a.group % 2 == 0) ? 2 : 1;
  if (head_dim == 64) {
    if (hpw == 4) return launch_hpw<64, 4>(a, stream);
    if (hpw == 2) return launch_hpw<64, 2>(a, stream);
    return launch_hpw<64, 1>(a, stream);
  }
  if (hpw == 4) return launch_hpw<128, 4>(a, stream);
  if (hpw == 2) return launch_hpw<128, 2>(a, stream);
  return launch_hpw<128, 1>(a, stream);
}

}  // namespace pa
