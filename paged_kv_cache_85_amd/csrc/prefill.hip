// Varlen causal prefill over a paged KV cache on the gfx950 matrix cores
// (bf16 inputs, fp32 accumulation).
//
// Prompts are packed end to end; each row sees its own prompt up to its own
// position ("mini-vLLM", project summary); sequence boundaries come from cu_seqlens_q / cu_seqlens_k, and
// cu_seqlens_k > cu_seqlens_q means the sequence already has a cached prefix
// (smzdm Nano-vLLM walk-through, model implementation details), so its Lq new
// rows are the last rows of the sequence: row i sees keys 0 .. Lk - Lq + i.
// All keys are read from the pools through the block table.
//
// Tiling.  A workgroup (4 waves) owns one KV head, HPW of its query heads and
// BMQ = 32 * (4 / HPW) consecutive query rows; each wave owns 32 rows of one
// head.  Key/value tiles of 32 tokens are gathered through the block table
// into LDS once per workgroup and shared by the four waves.  Per tile a wave
// computes
//     S^T (32 keys x 32 rows)  = K_tile . Q^T       (v_mfma_f32_32x32x16_bf16)
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
// Tile ring.  LDS holds three tile stages; tile kt + 2 is requested while tile
// kt is computed, and one barrier per tile both publishes the arrived tile
// and frees the stage the next request overwrites.  When a block holds whole
// tiles (power-of-two block size >= 32) the tiles travel from HBM straight
// into LDS (buffer loads with the LDS-destination bit: no register staging,
// no LDS store instructions); other block sizes look every row up on its own
// and pass it through registers.  Both loaders fill the same layout, so the
// arithmetic -- and the result, bit for bit -- does not depend on the block
// size.
//
// LDS rows are unpadded (D elements) and XOR-swizzled at 16-byte granularity:
// logical chunk c of row r sits at physical chunk c ^ swz(r), with swz chosen
// so that the 16 rows of an operand read and the 4 keys x 4 chunks of a
// transpose read each touch all 64 banks once.
//
// Work order: the grid runs the last (heaviest, under the causal mask) query
// tiles of every sequence first.  Tiles entirely above the diagonal are
// skipped; masking is applied only to tiles that cross it.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int swap_bits_2_3(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

#ifndef PA_PREFILL_OCC
#define PA_PREFILL_OCC 2
#endif

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (base, no stride, num_records = bytes) in scalar
// registers; offsets at or past `bytes` read zero.
__device__ __forceinline__ u32x4 stream_rsrc(const void* base, unsigned bytes) {
  const unsigned long long p = (unsigned long long)base;
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((unsigned)p),
               (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu),
               (unsigned)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// 16 bytes per lane from buffer offset voff straight into LDS: the wave's 64
// lanes fill 1 KiB at LDS byte address `lds` (wave-uniform) in lane order;
// NT adds the non-temporal cache policy (gfx940-family bit NT).  Issued as
// inline assembly so that the compiler does not add its own waits for it;
// the caller orders it with vm_wait and barriers.
template <bool NT>
__device__ __forceinline__ void lds_load16(u32x4 rsrc, unsigned lds, unsigned voff) {
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// Wait until at most N vector-memory loads of this thread are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS transpose read: within each 16-lane group, lane j points at 4
// consecutive 16-bit elements (chunk j); lane i receives element
// chunk[4k + i/4][i%4] as its k-th value.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Physical 16-byte chunk of logical chunk c in tile row r is c ^ tile_swz(r).
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

#ifndef PA_PREFILL_BN
#define PA_PREFILL_BN 32
#endif
#ifndef PA_PREFILL_NST
#define PA_PREFILL_NST 3
#endif
#ifndef PA_PREFILL_SPLIT
#define PA_PREFILL_SPLIT 0
#endif

// Wait until at most `tiles` tile requests of NI16 16-byte loads each are
// still in flight (0 <= tiles <= MAXT).
template <int PER_TILE, int MAXT>
__device__ __forceinline__ void wait_tiles(int tiles) {
  if constexpr (MAXT > 0) {
    if (tiles >= MAXT) {
      vm_wait<MAXT * PER_TILE>();
      return;
    }
    wait_tiles<PER_TILE, MAXT - 1>(tiles);
  } else {
    vm_wait<0>();
  }
}

// Persistent launches keep one 16-bit tile count per sequence in LDS.
constexpr int kMaxPersistSeqs = 2048;

// Position of a walk over the heavy-first item list, in chunks of 64
// sequences of one query-tile index: chunk (qt_rev, b0) starts at rank kbase
// among the non-empty items.
struct ItemWalk {
  int qt_rev;
  int b0;
  int kbase;
};

// Advance the walk to the non-empty item of rank k (k never decreases between
// calls); false once the list is exhausted.  Wave-uniform.
__device__ __forceinline__ bool walk_to(ItemWalk& wk, int k, const uint16_t* ntiles,
                                        int num_seqs, int n_qt, int inner, int lane, int& qt,
                                        int& b, int& gh) {
  while (wk.qt_rev < n_qt) {
    const int q = n_qt - 1 - wk.qt_rev;
    const int bb = wk.b0 + lane;
    const bool v = bb < num_seqs && (int)ntiles[bb] > q;
    const unsigned long long m = __ballot(v);
    const int cnt = __popcll(m) * inner;
    if (k < wk.kbase + cnt) {
      const int t = k - wk.kbase;
      const int s = t / inner;
      gh = t - s * inner;
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
      const unsigned long long sel = __ballot(v && below == s);
      b = wk.b0 + __builtin_ctzll(sel);
      qt = q;
      return true;
    }
    wk.kbase += cnt;
    wk.b0 += 64;
    if (wk.b0 >= num_seqs) {
      wk.b0 = 0;
      ++wk.qt_rev;
    }
  }
  return false;
}

// Cache policy of the key/value tiles.  Tiles of a sequence with several
// query rows are re-read through L2 by its other query tiles and heads; a
// decode row (one query row) reads each of its tiles once, so those stream
// with the non-temporal policy.
enum TilePolicy : int {
  kTilesCached = 0,    // every item: default policy
  kTilesStreamed = 1,  // every item is a decode row: non-temporal
  kTilesPerItem = 2,   // mixed batches: non-temporal for items of one query row
};

// BN keys per tile, NST tile stages in LDS, POL a TilePolicy.
template <int D, int HPW, bool DMA, int BN, int NST, int POL>
__global__ __launch_bounds__(256, PA_PREFILL_OCC) void prefill_bf16_kernel(
    PrefillArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k) {
  constexpr int NB = BN / 32;                // 32-key score blocks per tile
  constexpr int WPH = 4 / HPW;
  constexpr int BMQ = 32 * WPH;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NI = BN * CPR / 256;         // loads per thread per tensor per tile
  constexpr int SPLIT = (NB == 1 && PA_PREFILL_SPLIT) ? 2 : 1;
  static_assert(NST >= 2 && NST <= 4, "stage count");

  // Stage s: K rows [0, BN*D), then V rows.
  __shared__ __attribute__((aligned(16))) uint16_t st[NST][2 * BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31;
  const int lh = lane >> 5;

  const int num_seqs = a.num_seqs;
  const int hchunks = a.group / HPW;
  const int inner = a.num_kv_heads * hchunks;
  const int n_qt = (a.max_seqlen_q + BMQ - 1) / BMQ;

  // Work items, heaviest first: item ((qt_rev * num_seqs) + b) * inner + gh
  // is query tile n_qt - 1 - qt_rev of sequence b, KV head / head chunk gh;
  // tiles past a sequence's end are empty.  A launch with one workgroup per
  // item maps blockIdx to its item.  A persistent launch (one workgroup per
  // resident slot) walks the non-empty items in that order.  Workgroup i of G
  // first takes the item of rank i.  With a work counter, every later item
  // goes to whichever workgroup asks first -- heaviest first to the first
  // free workgroup, which evens out both the items' costs and the
  // workgroups' unequal speeds; each workgroup draws its next rank a few
  // tiles before its current item ends (its first wave waits for the draw
  // there: the compiler's wave-aggregated atomic reads the result at once).
  // A launch of G workgroups makes exactly G draws past the
  // end of the list, and the one that draws the last value puts the counter
  // back to zero.  Without a counter the ranks are dealt in a snake: r * G + i
  // (r even) or r * G + G - 1 - i (r odd).  Which workgroup computes an item
  // never changes its arithmetic.
  __shared__ uint16_t s_ntiles[kMaxPersistSeqs];
  __shared__ int s_items[4];
  __shared__ unsigned s_ticket;
  const bool persistent = a.persistent != 0;
  int n_items = 0;  // non-empty items (persistent launches)
  if (persistent) {
    int mine = 0;
    for (int i = tid; i < num_seqs; i += 256) {
      const int qs = cu_q[i], qe = cu_q[i + 1], kl = cu_k[i + 1] - cu_k[i];
      int nq = 0;
      if (qs >= 0 && qs < a.total_q) {
        const int lk = min(min(kl, a.max_seqlen_k), a.max_blocks_per_seq * a.block_size);
        const int lq = min(min(min(qe - qs, a.max_seqlen_q), lk), a.total_q - qs);
        nq = lq > 0 ? (lq + BMQ - 1) / BMQ : 0;
      }
      s_ntiles[i] = (uint16_t)nq;
      mine += nq;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off);
    if (lane == 0) s_items[w] = mine;
    __syncthreads();
    n_items = (s_items[0] + s_items[1] + s_items[2] + s_items[3]) * inner;
  }
  ItemWalk walk{0, 0, 0};
  const int G = gridDim.x;
  const int gi = blockIdx.x;
  // XCD groups.  The workgroups of a launch are placed on the chip's eight
  // XCDs in turn (workgroup i on XCD i mod 8), and each XCD has an L2 of its
  // own.  When the launcher asks for it (sequences of several query tiles,
  // which re-read their keys and values), with a work counter and a
  // KV-head/chunk count that is a multiple of 8, group x (the workgroups
  // i = x mod 8) deals among itself only the items of head/chunk
  // gh = x mod 8, heaviest first, through a counter of its own: the keys and
  // values a head's query tiles re-read then come from one L2, and every
  // group has the same work (heads cost the same).  The item order and
  // dealing within a group are those described above with G / 8 workgroups
  // and inner / 8 head/chunks.
  constexpr int kXcds = 8;
  const bool grouped = a.xcd_groups != 0 && persistent && a.ticket != nullptr &&
                       inner % kXcds == 0 && G % kXcds == 0;
  const int GX = grouped ? G / kXcds : G;          // workgroups dealing together
  const int gx = grouped ? gi / kXcds : gi;        // this workgroup among them
  const int xg = grouped ? gi % kXcds : 0;         // its group
  const int innerx = grouped ? inner / kXcds : inner;
  const int n_itemsx = grouped ? n_items / kXcds : n_items;
  // Group x's counter sits 32 bytes after group x - 1's: the eight fill the
  // 256-byte workspace.
  unsigned* const ticket = a.ticket != nullptr ? a.ticket + xg * 8 : nullptr;
  // Dynamic dealing needs every workgroup to hold a first item (each then
  // draws until a draw comes back past the end).
  const bool dyn = persistent && ticket != nullptr && n_itemsx > GX;
  const unsigned last_draw = (unsigned)(n_itemsx - GX) + (unsigned)GX - 1u;
  unsigned tk = 0;     // thread 0: the rank drawn during the current item
  bool drew = false;   // thread 0: whether that draw has been made

  for (int round = 0;; ++round) {
  int qt, b, gh;
  if (persistent) {
    int k;
    if (dyn && round > 0) {
      // The rank drawn during the previous item (drawn now if that item
      // ended before its draw point), published to the whole workgroup.
      if (tid == 0) {
        if (!drew) tk = atomicAdd(ticket, 1u);
        s_ticket = tk;
      }
      __syncthreads();
      const unsigned t = __builtin_amdgcn_readfirstlane(s_ticket);
      drew = false;
      if ((long)GX + t >= (long)n_itemsx) {
        if (t == last_draw && tid == 0)
          __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      k = GX + (int)t;
    } else {
      k = round * GX + ((round & 1) ? GX - 1 - gx : gx);
    }
    if (!walk_to(walk, k, s_ntiles, num_seqs, n_qt, innerx, lane, qt, b, gh)) break;
    gh = gh * (grouped ? kXcds : 1) + xg;
  } else {
    if (round > 0) break;
    int x = gi;
    gh = x % inner;
    x /= inner;
    b = x % num_seqs;
    qt = n_qt - 1 - x / num_seqs;
  }
  const int g = gh / hchunks;
  const int hc = gh % hchunks;

  // Sequence bounds: scalar loads (restrict, uniform address), kept uniform.
  const int q_start = __builtin_amdgcn_readfirstlane(cu_q[b]);
  const int q_end = __builtin_amdgcn_readfirstlane(cu_q[b + 1]);
  const int k_len = __builtin_amdgcn_readfirstlane(cu_k[b + 1] - cu_k[b]);
  if (q_start < 0 || q_start >= a.total_q) continue;
  const int Lk = min(min(k_len, a.max_seqlen_k), a.max_blocks_per_seq * a.block_size);
  const int Lq = min(min(min(q_end - q_start, a.max_seqlen_q), Lk), a.total_q - q_start);
  if (qt < 0 || qt * BMQ >= Lq) continue;
  const int delta = Lk - Lq;
  const float scale_log2 = a.scale_log2;
  const int num_q_heads = a.num_q_heads;

  const int head_local = w / WPH;
  const int h = g * a.group + hc * HPW + head_local;
  const int row0 = qt * BMQ + (w % WPH) * 32;
  const bool wave_active = row0 < Lq;
  const int kmax_wave = delta + min(row0 + 32, Lq) - 1;
  const int kmax_wg = delta + min(qt * BMQ + BMQ, Lq) - 1;
  const int n_tiles = kmax_wg / BN + 1;
  const int draw_kt = max(0, n_tiles - 3);  // tile step at which the next rank is drawn

  bf16x8 qB[KC];
  const uint16_t* kcache = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vcache = reinterpret_cast<const uint16_t*>(a.v_cache);
  const int32_t* bt = tables + (long)b * a.max_blocks_per_seq;
  const int slot_elems = a.num_kv_heads * D;
  const unsigned row_bytes = (unsigned)slot_elems * 2u;
  const int bs = a.block_size;
  const int bs_log2 = a.block_size_log2;
  const int nblk = a.num_blocks;
  // Byte addresses of this KV head's rows in the pools, and the bytes from
  // one block to the next: a tile's descriptor base is then one product and
  // two additions away.
  const char* khead = reinterpret_cast<const char*>(a.k_cache) + (long)g * D * 2;
  const char* vhead = reinterpret_cast<const char*>(a.v_cache) + (long)g * D * 2;
  const unsigned blk_bytes = (unsigned)bs * row_bytes;  // < 2^32 on this path (launcher)
  // LDS byte address of stage 0 (a constant of the kernel).
  const unsigned st_lds =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&st[0][0];

  // Load i of this wave fills physical chunks [(w * NI + i) * 64, +64) of a
  // tile: row s / CPR, physical chunk s % CPR, which holds logical chunk
  // (s % CPR) ^ swz(row).
  unsigned src_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s = (w * NI + i) * 64 + lane;
    const int r = s / CPR;
    const int c = (s % CPR) ^ tile_swz<D>(r);
    src_off[i] = (unsigned)r * row_bytes + (unsigned)(c * 16);
  }

  // Request tile kt, which lies in physical block blk_id, into LDS stage
  // `stage` (K rows, then V rows).  Rows past Lk lie outside the descriptors
  // and arrive as zeros.
  const bool stream_tiles = POL == kTilesStreamed || (POL == kTilesPerItem && Lq == 1);
  auto request = [&](int stage, int kt, int blk_id) __attribute__((always_inline)) {
    const int t0 = kt * BN;
    const int blk = clamp_block(blk_id, nblk);
    const unsigned long long off = (unsigned long long)(unsigned)blk * blk_bytes +
                                   (unsigned)(t0 & (bs - 1)) * row_bytes;
    const unsigned bytes = (unsigned)min(BN, Lk - t0) * row_bytes;
    const u32x4 rk = stream_rsrc(khead + off, bytes);
    const u32x4 rv = stream_rsrc(vhead + off, bytes);
    const unsigned dk = st_lds + (unsigned)(stage * 2 * BN * D * 2 + w * NI * 1024);
    const unsigned dv = dk + BN * D * 2;
    if (stream_tiles) {
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_load16<true>(rk, dk + i * 1024, src_off[i]);
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_load16<true>(rv, dv + i * 1024, src_off[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_load16<false>(rk, dk + i * 1024, src_off[i]);
#pragma unroll
      for (int i = 0; i < NI; ++i) lds_load16<false>(rv, dv + i * 1024, src_off[i]);
    }
  };

  // Other block sizes: the same chunks through registers, each row looked up
  // in the block table on its own, then written to the same LDS positions.
  uint4 kreg[NI], vreg[NI];
  auto fetch = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s = (w * NI + i) * 64 + lane;
      const int j = kt * BN + s / CPR;
      if (j < Lk) {
        long slot;
        if (bs_log2 >= 0)
          slot = ((long)clamp_block(bt[j >> bs_log2], nblk) << bs_log2) + (j & (bs - 1));
        else
          slot = (long)clamp_block(bt[j / bs], nblk) * bs + j % bs;
        const int c = (s % CPR) ^ tile_swz<D>(s / CPR);
        const long off = slot * slot_elems + (long)g * D + c * 8;
        kreg[i] = *reinterpret_cast<const uint4*>(kcache + off);
        vreg[i] = *reinterpret_cast<const uint4*>(vcache + off);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto deposit = [&](uint16_t* dk, uint16_t* dv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s = (w * NI + i) * 64 + lane;
      *reinterpret_cast<uint4*>(dk + s * 8) = kreg[i];
      *reinterpret_cast<uint4*>(dv + s * 8) = vreg[i];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.f;
  const int my_row = row0 + lr;
  const int klim = delta + my_row;
  // K operand: lane reads tile row 32 * nb + krow (bits 2 and 3 of lr
  // swapped) at logical chunk 2 * kk + lh.
  const int krow = swap_bits_2_3(lr);
  const int kswz = tile_swz<D>(krow);
  // V transpose operand: lane reads key 16 * kc + 8 * lh + 4 * half + j / 4,
  // elements 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3) .. + 3.
  const int tr_j = lane & 15;
  const int tr_key = 8 * lh + tr_j / 4;
  const int tr_el = 16 * ((lane >> 4) & 1) + 4 * (tr_j & 3);

  auto compute = [&](const uint16_t* sk, const uint16_t* sv, int kt) __attribute__((always_inline)) {
    f32x16 sacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // (tile_swz of rows 32 * nb + krow equals that of krow: it only reads
      // the low four bits of the row.)
      if constexpr (SPLIT == 2) {
        f32x16 s2[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const int pc = (2 * kk + lh) ^ kswz;
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(sk + (nb * 32 + krow) * D + pc * 8);
          s2[kk & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qB[kk], s2[kk & 1], 0, 0, 0);
        }
        sacc[nb] = s2[0] + s2[1];
      } else {
        sacc[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const int pc = (2 * kk + lh) ^ kswz;
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(sk + (nb * 32 + krow) * D + pc * 8);
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qB[kk], sacc[nb], 0, 0, 0);
        }
      }
    }
    // Item t of block nb holds the raw score of key
    // kt*BN + 32*nb + 16*(t/8) + 8*lh + t%8.
    const bool need_mask = (kt * BN + BN - 1 > delta + row0) || (kt * BN + BN > Lk);
    if (need_mask) {
      // Key kt*BN + 8*lh + off is visible iff it is <= klim and < Lk, i.e.
      // iff off <= min(klim, Lk - 1) - kt*BN - 8*lh.
      const int thr = min(klim, Lk - 1) - (kt * BN + 8 * lh);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int t = 0; t < 16; ++t)
          if (32 * nb + 16 * (t >> 3) + (t & 7) > thr) sacc[nb][t] = -INFINITY;
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, sacc[nb][t]);
    mx = xor_max<32>(mx) * scale_log2;  // scale > 0: max commutes with it
    // Lazy rescale: the reference max m_run only moves when a row's max
    // exceeds it by more than 2^8 (so probabilities stay <= 256); the final
    // O / l is the same for any reference, and the O rescale is skipped for
    // every tile that does not move it.
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
    bf16x8 pB[2 * NB];
#pragma unroll
    for (int kc = 0; kc < 2 * NB; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = fast_exp2(fmaf(sacc[kc >> 1][(kc & 1) * 8 + e], scale_log2, -m_run));
        psum += pr;
        pB[kc][e] = (__bf16)pr;
      }
    }
    l_run += psum;
#pragma unroll
    for (int kc = 0; kc < 2 * NB; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 part[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int key = kc * 16 + tr_key + 4 * half;
          const int el = db * 32 + tr_el;
          const int pc = (el >> 3) ^ tile_swz<D>(key);
          part[half] = lds_read_tr(sv + key * D + pc * 8 + (el & 7));
        }
        const bf16x8 A = {part[0][0], part[0][1], part[0][2], part[0][3],
                          part[1][0], part[1][1], part[1][2], part[1][3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, pB[kc], oacc[db], 0, 0, 0);
      }
    }
  };

  int blk_next = 0;  // physical block of the next DMA request
  if constexpr (DMA) {
    if (NST - 1 < n_tiles) blk_next = bt[((NST - 1) * BN) >> bs_log2];
  }

  // One tile step on stage S = kt % NST: wait for this thread's requests of
  // tile kt (later tiles' requests may stay in flight), publish them with the
  // barrier -- which also tells every wave that stage (kt - 1) % NST, read
  // during tile kt - 1, is free -- request tile kt + NST - 1 into it, compute.
  auto step = [&](auto stage, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    uint16_t* sk = st[S];
    uint16_t* nk = st[(S + NST - 1) % NST];
    uint16_t* sv = sk + BN * D;
    uint16_t* nv = nk + BN * D;
    // (The draw is one more vector-memory operation in flight for wave 0;
    // the tile waits below then wait for one operation more than needed,
    // never fewer, since operations complete in issue order.)
    if (dyn && tid == 0 && kt == draw_kt) {
      tk = atomicAdd(ticket, 1u);
      drew = true;
    }
    if constexpr (DMA) {
      wait_tiles<2 * NI, NST - 2>(min(NST - 2, n_tiles - 1 - kt));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NST - 1 < n_tiles) {
        request((S + NST - 1) % NST, kt + NST - 1, blk_next);
        // The block of the next request is loaded a step ahead, so that the
        // wave never waits on the block table.
        if (kt + NST < n_tiles) blk_next = bt[((kt + NST) * BN) >> bs_log2];
      }
      if (wave_active && kt * BN <= kmax_wave) compute(sk, sv, kt);
    } else {
      __syncthreads();
      if (kt + NST - 1 < n_tiles) fetch(kt + NST - 1);
      if (wave_active && kt * BN <= kmax_wave) compute(sk, sv, kt);
      if (kt + NST - 1 < n_tiles) deposit(nk, nv);
    }
  };

#pragma unroll
  for (int t = 0; t < NST - 1; ++t) {
    if (t < n_tiles) {
      if constexpr (DMA) {
        request(t, t, bt[(t * BN) >> bs_log2]);
      } else {
        fetch(t);
        deposit(st[t], st[t] + BN * D);
      }
    }
  }
  {
    const int qrow = row0 + lr;
    if (wave_active && qrow < Lq) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           ((long)(q_start + qrow) * num_q_heads + h) * D + lh * 8;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qB[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
    } else {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) qB[kk] = bf16x8{};
    }
  }
  // The first tiles and Q are needed before any work: wait for everything
  // here, so that no later wait for Q (which would also drain the tiles in
  // flight) is needed inside the loop.
  vm_wait<0>();

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  for (int kt = 0; kt < n_tiles; kt += NST) {
    step(I0{}, kt);
    if (kt + 1 >= n_tiles) break;
    step(I1{}, kt + 1);
    if constexpr (NST > 2) {
      if (kt + 2 >= n_tiles) break;
      step(I2{}, kt + 2);
    }
    if constexpr (NST > 3) {
      if (kt + 3 >= n_tiles) break;
      step(I3{}, kt + 3);
    }
  }

  const float l_tot = xor_sum<32>(l_run);
  if (wave_active) {
    const float inv = 1.f / l_tot;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                   ((long)(q_start + my_row) * num_q_heads + h) * D;
    // Item t of block db is head-dim element db*32 + 8*(t/4) + 4*lh + t%4:
    // per 16 elements db*32 + 16*j .. + 15, the lane of half lh = 0 holds
    // the quarters 0 and 2, its partner 32 lanes up the quarters 1 and 3.
    // One lane swap per dword gives the lower lane the first 8 elements and
    // its partner the last 8, so each stores 16 contiguous bytes.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned w[2][2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int t = (2 * j + q) * 4;
          w[q][0] = pack_bf16x2(oacc[db][t + 0] * inv, oacc[db][t + 1] * inv);
          w[q][1] = pack_bf16x2(oacc[db][t + 2] * inv, oacc[db][t + 3] * inv);
        }
        uint4 u;
        const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
        u.x = s0[0];
        u.y = s1[0];
        u.z = s0[1];
        u.w = s1[1];
        if (my_row < Lq) *reinterpret_cast<uint4*>(op + db * 32 + 16 * j + 8 * lh) = u;
      }
    }
  }
  // Every wave is done with the LDS stages before the next item refills them.
  __syncthreads();
  }
}

// Persistent launches keep one 16-bit query-tile count per sequence in LDS:
// at most kMaxPersistSeqs sequences, each of at most 0xffff query tiles.
static bool persistent_ok(const PrefillArgs& a, long long n_items, int slots, int bmq) {
  return a.num_seqs <= kMaxPersistSeqs &&
         ((long long)a.max_seqlen_q + bmq - 1) / bmq <= 0xffff && n_items > slots;
}

// XCD groups pay off when the sequences average two query tiles or more
// (their later tiles re-read the keys and values of the earlier ones).
// Batches of mostly decode rows read every tile once, and there eight
// separate pools of items of unequal, unsorted cost only lengthen the tail
// (decode rows as one launch: 226 us grouped against 210 us).
static bool xcd_groups_ok(const PrefillArgs& a, int bmq) {
  return (long long)a.total_q >= 2LL * bmq * a.num_seqs;
}

template <int D, int HPW, bool DMA, int POL>
static int launch_items(const PrefillArgs& a, long long n_items, hipStream_t stream) {
  constexpr int BN = PA_PREFILL_BN;
  constexpr int NST = PA_PREFILL_NST;
  constexpr int BMQ = 32 * (4 / HPW);
  static std::atomic<int> slots_cache[kMaxDevices];
  const int slots = resident_blocks(
      reinterpret_cast<const void*>(prefill_bf16_kernel<D, HPW, DMA, BN, NST, POL>), 256,
      slots_cache);
  if (slots < 0) return -1;
  PrefillArgs p = a;
  p.persistent = persistent_ok(a, n_items, slots, BMQ) ? 1 : 0;
  p.xcd_groups = xcd_groups_ok(a, BMQ) ? 1 : 0;
  const long long grid = p.persistent ? slots : n_items;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, HPW, DMA, BN, NST, POL>), dim3((unsigned)grid),
                     dim3(256), 0, stream, p, a.block_tables, a.cu_seqlens_q, a.cu_seqlens_k);
  return 0;
}

template <int D, int HPW>
static int launch_hpw(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BMQ = 32 * (4 / HPW);
  const long long n_qt = (a.max_seqlen_q + BMQ - 1) / BMQ;
  const long long n_items =
      n_qt * a.num_seqs * (long long)a.num_kv_heads * (a.group / HPW);
  if (n_items <= 0) return 0;
  if (n_items > 0x7fffffffLL) return -1;
  const long long row_bytes = (long long)a.num_kv_heads * D * 2;
  if (a.block_size_log2 >= 0 && (1 << a.block_size_log2) >= PA_PREFILL_BN &&
      (1LL << a.block_size_log2) * row_bytes < (1LL << 32)) {
    // Tiles inside one block.  When every query row is a decode row (one
    // row per sequence), each key/value tile is read by a single item:
    // those launches stream the tiles past the caches, as decode does; any
    // longer query tile re-reads its sequence's tiles through L2.  A batch
    // whose sequences average less than one query tile each is taken for
    // a mixed one (decode rows beside a few prompts): its items choose
    // their policy one by one.  (Per-item choice on prompt-only batches
    // measured 2.5 % slower on the prefix-cache workload, so they keep one
    // policy for the launch.)
    if (a.max_seqlen_q == 1)
      return launch_items<D, HPW, true, kTilesStreamed>(a, n_items, stream);
    if ((long long)a.total_q < (long long)BMQ * a.num_seqs)
      return launch_items<D, HPW, true, kTilesPerItem>(a, n_items, stream);
    return launch_items<D, HPW, true, kTilesCached>(a, n_items, stream);
  }
  return launch_items<D, HPW, false, kTilesCached>(a, n_items, stream);
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
