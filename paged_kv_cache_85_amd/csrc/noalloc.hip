// pa_decode_noalloc: pa_decode for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation).  Its split-context workspace is a file-scope device
// array of PA_NOALLOC_SCRATCH_BYTES bytes: the code object holds one copy per
// GPU, from the moment the library is loaded on that GPU until the process
// ends.  The call itself allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"
#include "device_common.h"
#include "pa_internal.h"

namespace {

// The decode work counter (first 256 bytes) and the partial results.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

// The counter must read zero when a decode call starts.  Every call leaves it
// zero, but a fill kernel (not a memset node, which stream capture must not
// record) clears it on the caller's stream before each call that uses it, so
// a call never depends on what an earlier, possibly unfinished, call left.
__global__ __launch_bounds__(64) void clear_counter_kernel(unsigned* counter) {
  counter[threadIdx.x] = 0u;
}

// Device address of each GPU's copy of `scratch`.  In host code the name
// `scratch` is a host-side stand-in, not a device address: only the address
// returned by hipGetSymbolAddress, taken with that device current, may be
// passed to kernels.
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[pa::kMaxDevices];

void* scratch_of_current_device(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pa::kMaxDevices) {
    *status = PA_E_HIP;
    return nullptr;
  }
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess) d.ptr = p;
  });
  if (d.err != hipSuccess || !d.ptr) {
    *status = PA_E_HIP;
    return nullptr;
  }
  *status = PA_OK;
  return d.ptr;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_blocks, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t dtype, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need =
      pa::decode_scratch_need(num_seqs, num_q_heads, head_dim, max_context_len);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    int status = PA_OK;
    ws = scratch_of_current_device(&status);
    if (!ws) return status;
    // (A call that then fails its argument checks has only cleared a counter.)
    hipLaunchKernelGGL(clear_counter_kernel, dim3(1), dim3(64), 0, s,
                       static_cast<unsigned*>(ws));
    if (hipGetLastError() != hipSuccess) return PA_E_HIP;
  }
  return pa::decode_entry(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq, max_context_len, scale, dtype, ws,
                          ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, s);
}
