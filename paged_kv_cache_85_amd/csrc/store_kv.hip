// K/V store: scatter each new token's K and V row into its pool slot.
//
// The store writes K/V for every new prompt token in prefill and one token
// per sequence in decode ("nano-vLLM Part 4", section 3, prefill/decode
// table); the slot mapping names each row's physical position (smzdm
// Nano-vLLM walk-through, model implementation details).
//
// A token row is num_kv_heads * head_dim contiguous elements both in k/v and
// in the pool (the pool is [blocks, block_size, kv_heads, head_dim]), so the
// store is a row copy.  Lanes of a row take consecutive VEC-byte chunks, so
// every load and store instruction is fully coalesced; K and V are copied by
// the same thread to keep two independent streams in flight.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

template <int VEC>
struct Chunk;
template <>
struct Chunk<16> { typedef uint4 type; };
template <>
struct Chunk<8> { typedef uint2 type; };
template <>
struct Chunk<4> { typedef uint32_t type; };
template <>
struct Chunk<2> { typedef uint16_t type; };

// blockDim.x = 256.  A row is covered by `tpr` threads (a power of two,
// <= 256) which step over its `cpr` chunks; a block handles 256 / tpr rows.
template <int VEC>
__global__ __launch_bounds__(256) void store_kv_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int num_tokens,
    int cpr, int tpr_log2, long long num_slots) {
  typedef typename Chunk<VEC>::type C;
  const int tpr = 1 << tpr_log2;
  const int rows_per_block = 256 >> tpr_log2;
  const long long t = (long long)blockIdx.x * rows_per_block + (threadIdx.x >> tpr_log2);
  if (t >= num_tokens) return;
  const long long slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding row, or out of range
  const long long row_bytes = (long long)cpr * VEC;
  const C* ks = reinterpret_cast<const C*>(k + t * row_bytes);
  const C* vs = reinterpret_cast<const C*>(v + t * row_bytes);
  C* kd = reinterpret_cast<C*>(k_cache + slot * row_bytes);
  C* vd = reinterpret_cast<C*>(v_cache + slot * row_bytes);
  for (int c = threadIdx.x & (tpr - 1); c < cpr; c += tpr) {
    C a = ks[c];
    C b = vs[c];
    kd[c] = a;
    vd[c] = b;
  }
}

int launch_store_kv(const void* k, const void* v, void* k_cache, void* v_cache,
                    const int32_t* slot_mapping, int num_tokens, long long row_bytes,
                    long long num_slots, hipStream_t stream) {
  const uintptr_t align = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                          reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | (uintptr_t)row_bytes;
  int vec = 16;
  while (vec > 1 && (align & (vec - 1))) vec >>= 1;
  if (vec < 2) return -1;  // rows are whole 2- or 4-byte elements
  const long long cpr = row_bytes / vec;
  int tpr_log2 = 0;
  while ((1LL << tpr_log2) < cpr && tpr_log2 < 8) ++tpr_log2;
  const int rows_per_block = 256 >> tpr_log2;
  const int grid = (num_tokens + rows_per_block - 1) / rows_per_block;
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  char* kp = static_cast<char*>(k_cache);
  char* vp = static_cast<char*>(v_cache);
  switch (vec) {
    case 16:
      hipLaunchKernelGGL(store_kv_kernel<16>, dim3(grid), dim3(256), 0, stream, kc, vc, kp, vp,
                         slot_mapping, num_tokens, (int)cpr, tpr_log2, num_slots);
      break;
    case 8:
      hipLaunchKernelGGL(store_kv_kernel<8>, dim3(grid), dim3(256), 0, stream, kc, vc, kp, vp,
                         slot_mapping, num_tokens, (int)cpr, tpr_log2, num_slots);
      break;
    case 4:
      hipLaunchKernelGGL(store_kv_kernel<4>, dim3(grid), dim3(256), 0, stream, kc, vc, kp, vp,
                         slot_mapping, num_tokens, (int)cpr, tpr_log2, num_slots);
      break;
    default:
      hipLaunchKernelGGL(store_kv_kernel<2>, dim3(grid), dim3(256), 0, stream, kc, vc, kp, vp,
                         slot_mapping, num_tokens, (int)cpr, tpr_log2, num_slots);
      break;
  }
  return 0;
}

}  // namespace pa
