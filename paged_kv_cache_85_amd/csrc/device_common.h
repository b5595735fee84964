// Device helpers shared by the gfx950 kernels of libpa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A bf16 element is the upper half of an fp32 word, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

// DPP lane permutations inside a 16-lane row (GFX9 encodings).
enum : int {
  DPP_QUAD_1032 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
  DPP_QUAD_2301 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i <-> 7 - i inside each 8-lane half row
  DPP_ROW_MIRROR = 0x140,     // lane i <-> 15 - i inside each 16-lane row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Lane i together with lane i ^ OFF (OFF = 16 or 32) through the gfx950
// lane-swap instructions, register to register: swapping x with itself
// leaves, in every lane, x of the lower-numbered partner in `a` and x of the
// higher-numbered one in `b`.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  static_assert(OFF == 16 || OFF == 32, "swap distance");
  const unsigned u = __float_as_uint(x);
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// x combined with x of lane i ^ OFF (OFF a power of two below 64): the same
// two operands as x + __shfl_xor(x, OFF) (or the max), so the same bits.
template <int OFF>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (OFF == 16 || OFF == 32) {
    float a, b;
    lane_pair<OFF>(x, a, b);
    return a + b;
  } else {
    return x + __shfl_xor(x, OFF);
  }
}
template <int OFF>
__device__ __forceinline__ float xor_max(float x) {
  if constexpr (OFF == 16 || OFF == 32) {
    float a, b;
    lane_pair<OFF>(x, a, b);
    return fmaxf(a, b);
  } else {
    return fmaxf(x, __shfl_xor(x, OFF));
  }
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a group
// receives the group total.  After the two quad steps each quad holds its own
// sum; the half-row mirror pairs the two quads of an 8-lane half; the row
// mirror pairs the two halves of a 16-lane row; a 32-lane group adds the
// neighbouring row with a lane swap.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<DPP_QUAD_1032>(x);
  x += dpp<DPP_QUAD_2301>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x = xor_sum<16>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Finite stand-in for "no score seen yet": exp2(kNegBig - m) is 0 for any
// real score m, and exp2(kNegBig - kNegBig) is 1, so no NaN arises.
constexpr float kNegBig = -1.0e30f;

// Context partitions of a row of L tokens (P tokens each).
__device__ __forceinline__ int num_parts(int L, int P) { return L > 0 ? (L + P - 1) / P : 0; }

__device__ __forceinline__ int clamp_block(int blk, int num_blocks) {
  return min(max(blk, 0), num_blocks - 1);
}

// Persistent launches size their grid as CUs x resident blocks per CU of the
// kernel, queried once per device and kept in `cache` (one table per kernel;
// zero means not known yet).  Host threads that ask for the first time
// together may each query the runtime; they store the same value, so the
// table needs no lock.  Devices past kMaxDevices are queried on every call.
constexpr int kMaxDevices = 64;

// SIMDs of the current device (4 per CU on this architecture), cached like
// resident_blocks.
inline int device_simds(std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  const int v = 4 * (cus > 0 ? cus : 1);
  if (cached) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

inline int resident_blocks(const void* kernel, int threads, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return -1;
  const int v = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  if (cached) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace pa
