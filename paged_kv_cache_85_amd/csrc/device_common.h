// Device helpers shared by the gfx950 kernels of libpa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a group
// receives the group total.  After the two quad steps each quad holds its own
// sum; the half-row mirror pairs the two quads of an 8-lane half; the row
// mirror pairs the two halves of a 16-lane row; a 32-lane group adds the
// neighbouring row through ds_swizzle/bpermute.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<DPP_QUAD_1032>(x);
  x += dpp<DPP_QUAD_2301>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Finite stand-in for "no score seen yet": exp2(kNegBig - m) is 0 for any
// real score m, and exp2(kNegBig - kNegBig) is 1, so no NaN arises.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int clamp_block(int blk, int num_blocks) {
  return min(max(blk, 0), num_blocks - 1);
}

}  // namespace pa
