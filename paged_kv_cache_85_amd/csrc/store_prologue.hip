// Store prologue: normalise each query and key head row by its RMS (with a
// learned per-element gain), rotate it by its token's position, and store the
// key and value rows into their pool slots -- one pass over the new tokens.
//
// Qwen3 normalises queries and keys per head before attention (smzdm
// Nano-vLLM walk-through, model implementation details); the model rotates
// queries and keys by position ("mini-vLLM", project summary: rotary
// embeddings); K/V then go to the slot the slot mapping names ("nano-vLLM
// Part 4", section 3).  The rotation is the half-split form: element i pairs
// with element i + D/2, both rotated by the angle of frequency i, whose cos
// and sin the caller supplies per position.
//
// A head row is D contiguous elements; LPH lanes each hold one 16-byte chunk,
// so a row is one coalesced access and its sum of squares is a DPP reduction
// over the LPH lanes.  The rotation partner of chunk c is chunk c ^ (LPH/2),
// one lane exchange away.  Arithmetic is fp32; the result is rounded once to
// the storage type.  Rows of one token are q heads, then k heads, then v
// heads (copied as they are).
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

template <typename T>
struct PrologueElem;
template <>
struct PrologueElem<float> {
  static constexpr int EPL = 4;
  __device__ static __forceinline__ void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static __forceinline__ uint4 narrow(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <>
struct PrologueElem<uint16_t> {
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
  __device__ static __forceinline__ uint4 narrow(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// blockDim.x = 256: 256 / LPH head rows per block, row r = token * R + j with
// R = Hq + 2 * Hkv.
template <typename T, int D>
__global__ __launch_bounds__(256) void store_prologue_kernel(PrologueArgs a) {
  typedef PrologueElem<T> E;
  constexpr int EPL = E::EPL;
  constexpr int LPH = D / EPL;  // lanes per head row
  constexpr int HALF = LPH / 2;
  static_assert(LPH == 8 || LPH == 16 || LPH == 32, "head row lanes");

  const int R = a.num_q_heads + 2 * a.num_kv_heads;
  const long long row = (long long)blockIdx.x * (256 / LPH) + threadIdx.x / LPH;
  const int c = threadIdx.x % LPH;
  if (row >= (long long)a.num_tokens * R) return;  // whole groups leave together
  const long long t = row / R;
  const int j = (int)(row - t * R);
  const long long slot = a.slot_mapping[t];
  const bool stored = slot >= 0 && slot < a.num_slots;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;

  if (j >= hq + hkv) {  // value head: copied as it is
    const int h = j - hq - hkv;
    if (stored) {
      const uint4 x = reinterpret_cast<const uint4*>(
          reinterpret_cast<const T*>(a.v) + (t * hkv + h) * D)[c];
      reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.v_cache) + (slot * hkv + h) * D)[c] = x;
    }
    return;
  }
  const bool is_q = j < hq;
  const int h = is_q ? j : j - hq;
  const T* src = is_q ? reinterpret_cast<const T*>(a.q) + (t * hq + h) * D
                      : reinterpret_cast<const T*>(a.k) + (t * hkv + h) * D;
  const T* gain = reinterpret_cast<const T*>(is_q ? a.q_weight : a.k_weight);
  const int pos = min(max(a.positions[t], 0), a.max_position - 1);
  const float* cs = a.cos_sin + (long long)pos * D + (c % HALF) * EPL;

  float x[EPL], w[EPL], cv[EPL], sv[EPL];
  E::widen(reinterpret_cast<const uint4*>(src)[c], x);
  E::widen(reinterpret_cast<const uint4*>(gain)[c], w);
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    const float4 cc = *reinterpret_cast<const float4*>(cs + e);
    const float4 ss = *reinterpret_cast<const float4*>(cs + D / 2 + e);
    cv[e] = cc.x; cv[e + 1] = cc.y; cv[e + 2] = cc.z; cv[e + 3] = cc.w;
    sv[e] = ss.x; sv[e + 1] = ss.y; sv[e + 2] = ss.z; sv[e + 3] = ss.w;
  }
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) sq = fmaf(x[e], x[e], sq);
  sq = group_sum<LPH>(sq);
  const float inv = 1.f / sqrtf(sq * (1.f / D) + a.eps);
  float y[EPL], o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) y[e] = x[e] * inv * w[e];
  const bool first = c < HALF;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float p = __shfl_xor(y[e], HALF);  // the element D/2 away
    o[e] = first ? fmaf(y[e], cv[e], -p * sv[e]) : fmaf(y[e], cv[e], p * sv[e]);
  }
  const uint4 out = E::narrow(o);
  if (is_q) {
    reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.q_out) + (t * hq + h) * D)[c] = out;
  } else if (stored) {
    reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.k_cache) + (slot * hkv + h) * D)[c] = out;
  }
}

template <typename T>
static int launch_typed(const PrologueArgs& a, int head_dim, hipStream_t stream) {
  const int lph = head_dim / (16 / (int)sizeof(T));
  const long long rows = (long long)a.num_tokens * (a.num_q_heads + 2 * a.num_kv_heads);
  const long long blocks = (rows + 256 / lph - 1) / (256 / lph);
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffffLL) return -1;
  if (head_dim == 64)
    hipLaunchKernelGGL((store_prologue_kernel<T, 64>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((store_prologue_kernel<T, 128>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  return 0;
}

int launch_store_prologue(const PrologueArgs& a, int head_dim, int dtype_bf16,
                          hipStream_t stream) {
  return dtype_bf16 ? launch_typed<uint16_t>(a, head_dim, stream)
                    : launch_typed<float>(a, head_dim, stream);
}

}  // namespace pa
