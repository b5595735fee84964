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
// heads (copied as they are); the cos/sin row of a position and the gains
// are read once per token, not once per head row.
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

// One wave per token (four tokens per 256-thread block).  Each lane loads
// the cos/sin values and the two gain vectors of its chunk once per token,
// then walks the token's R = Hq + 2 * Hkv head rows, 64 / LPH rows per
// instruction and U instructions' loads in flight before any arithmetic.
// All lanes of one LPH group work on the same row, so the group's reductions
// and the rotary partner exchange only read lanes of that row.
template <typename T, int D>
__global__ __launch_bounds__(256) void store_prologue_kernel(PrologueArgs a) {
  typedef PrologueElem<T> E;
  constexpr int EPL = E::EPL;
  constexpr int LPH = D / EPL;  // lanes per head row
  constexpr int HALF = LPH / 2;
  constexpr int RPI = 64 / LPH;  // rows per wave instruction
  constexpr int U = 4;           // instructions' rows loaded before computing
  static_assert(LPH == 8 || LPH == 16 || LPH == 32, "head row lanes");

  const long long t = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.num_tokens) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  const int c = lane % LPH;
  const int r = lane / LPH;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int R = hq + 2 * hkv;
  const long long slot = a.slot_mapping[t];
  const bool stored = slot >= 0 && slot < a.num_slots;
  const int pos = min(max(a.positions[t], 0), a.max_position - 1);
  const bool first = c < HALF;

  // Per-token constants of this lane's chunk.
  float cv[EPL], sv[EPL], wq[EPL], wk[EPL];
  {
    const float* cs = a.cos_sin + (long long)pos * D + (c % HALF) * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 cc = *reinterpret_cast<const float4*>(cs + e);
      const float4 ss = *reinterpret_cast<const float4*>(cs + D / 2 + e);
      cv[e] = cc.x; cv[e + 1] = cc.y; cv[e + 2] = cc.z; cv[e + 3] = cc.w;
      sv[e] = ss.x; sv[e + 1] = ss.y; sv[e + 2] = ss.z; sv[e + 3] = ss.w;
    }
    E::widen(reinterpret_cast<const uint4*>(a.q_weight)[c], wq);
    E::widen(reinterpret_cast<const uint4*>(a.k_weight)[c], wk);
  }
  const T* qrow = reinterpret_cast<const T*>(a.q) + t * hq * D;
  const T* krow = reinterpret_cast<const T*>(a.k) + t * hkv * D;
  const T* vrow = reinterpret_cast<const T*>(a.v) + t * hkv * D;

  for (int j0 = 0; j0 < R; j0 += RPI * U) {
    uint4 xr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RPI + r;
      if (j < hq) xr[u] = reinterpret_cast<const uint4*>(qrow + j * D)[c];
      else if (j < hq + hkv) xr[u] = reinterpret_cast<const uint4*>(krow + (j - hq) * D)[c];
      else if (j < R) xr[u] = reinterpret_cast<const uint4*>(vrow + (j - hq - hkv) * D)[c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RPI + r;
      if (j >= R) continue;
      if (j >= hq + hkv) {  // value head: copied as it is
        if (stored)
          reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.v_cache) +
                                   (slot * hkv + (j - hq - hkv)) * D)[c] = xr[u];
        continue;
      }
      const bool is_q = j < hq;
      float x[EPL];
      E::widen(xr[u], x);
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) sq = fmaf(x[e], x[e], sq);
      sq = group_sum<LPH>(sq);
      const float inv = 1.f / sqrtf(sq * (1.f / D) + a.eps);
      float y[EPL], o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) y[e] = x[e] * inv * (is_q ? wq[e] : wk[e]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float p = __shfl_xor(y[e], HALF);  // the element D/2 away
        o[e] = first ? fmaf(y[e], cv[e], -p * sv[e]) : fmaf(y[e], cv[e], p * sv[e]);
      }
      const uint4 out = E::narrow(o);
      if (is_q) {
        reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.q_out) + (t * hq + j) * D)[c] = out;
      } else if (stored) {
        reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.k_cache) + (slot * hkv + (j - hq)) * D)[c] =
            out;
      }
    }
  }
}

template <typename T>
static int launch_typed(const PrologueArgs& a, int head_dim, hipStream_t stream) {
  const long long blocks = ((long long)a.num_tokens + 3) / 4;
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
