// pa_decode_noalloc: pa_decode with its partial results in a fixed device array of the library's
// own, for callers that cannot allocate device memory (code under graph capture, serving loops
// that forbid hipMalloc). Plan, kernels and result bits are pa_decode's.
//
// The array `scratch` below exists once per GPU (each device holds its own copy at its own
// address, for the life of the process). In host code its name is only a host-side stand-in, so
// the device address is looked up with hipGetSymbolAddress, once per device with that device
// current, on the first call that needs it, and that address is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_launch.h"

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int num_seqs, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, float scale,
                                 pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                                 const float* k_scale, const float* v_scale, int partition_tokens,
                                 int variant, int flags, void* stream) {
  // the array used is the current device's: a stream of another device would have its kernels
  // read and write that device's address on a different GPU
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    int cur = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess ||
        hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_INVALID_ARG;
    }
    if (sdev != cur) return PA_ERR_INVALID_ARG;
  }
  return pa::decode_with_library_workspace(
      out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
      head_dim, block_size, max_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype, out_dtype,
      k_scale, v_scale, partition_tokens, variant, flags, PA_NOALLOC_SCRATCH_BYTES,
      scratch_address, stream);
}
