// Internal launch entry points of libpagedattn (host side). Each enqueues its kernels on the
// given stream and returns hipGetLastError(); all arguments were validated by pa_api.cpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Events the next kernel launch of this thread hands to the runtime, which stamps them at that
// kernel's own start and end (hipExtLaunchKernel); both null: a plain launch. The profiler in
// pa_api.cpp sets them around a pa_* call's one kernel; the launch clears them.
struct DispatchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
DispatchEvents& dispatch_events();

// Every kernel of the library is launched through this.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t st,
                          Args... args) {
  DispatchEvents& pending = dispatch_events();
  const DispatchEvents ev = pending;
  pending = DispatchEvents{};
  hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev.start, ev.stop, 0u, args...);
}

// pa_decode_append on a 1-D grid of grid_x work-groups: appends the work-groups that write the
// new tokens into the cache (one per 1024 (sequence, kv head, 8-dim piece) items; the hardware
// dispatches them after all the attention's, so they run in the launch's drain) and returns the
// grown grid. Plain decode, or a grid that would outgrow the launch limit, keeps grid_x and
// tail_wgs = 0 (then the attention's own work-groups write).
inline unsigned add_tail_writers(DecodeArgs& a, unsigned grid_x, int head_dim) {
  a.tail_from = 0;
  a.tail_wgs = 0;
  if (a.new_slots == nullptr) return grid_x;
  const long long pieces = static_cast<long long>(a.num_seqs) * a.num_kv_heads * (head_dim / 8);
  const long long wgs = (pieces + 1023) / 1024;
  if (static_cast<long long>(grid_x) + wgs > 0xFFFFFFFFLL / 256) return grid_x;
  a.tail_from = static_cast<int>(grid_x);
  a.tail_wgs = static_cast<int>(wgs);
  return grid_x + static_cast<unsigned>(wgs);
}

hipError_t launch_decode_valu(const DecodeArgs& a, int cache_dt, int q_dt, int head_dim,
                              int block_size, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeArgs& a, int cache_dt, int q_dt, int head_dim,
                              int block_size, hipStream_t st);
// Work-groups per CU the balanced MFMA kernel keeps resident, whatever its cache policy (0 if
// unknown).
int mfma_groups_per_cu(int cache_dt, int q_dt, int head_dim, int block_size, int group,
                       int num_seqs);
hipError_t launch_prefill(const PrefillArgs& a, int cache_dt, int q_dt, int head_dim, int block_size,
                          int max_query_len, hipStream_t st);
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int block_size, hipStream_t st);

hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int in_dt, int cache_dt,
                           const float* k_scale, const float* v_scale, hipStream_t st);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int num_pairs, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks, int cache_dt,
                              hipStream_t st);
hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const float* src_ks, const float* src_vs, float* dst_ks,
                              float* dst_vs, const int32_t* pairs, int num_pairs, int src_nb,
                              int dst_nb, int Hkv, int D, int B, int cache_dt, hipStream_t st);
// pa_decode's host logic (validation, plan, launches) with a workspace the library provides:
// every scalar check runs first; then, if the plan needs more than workspace_bytes, the call
// returns PA_ERR_WORKSPACE, and otherwise resolve_workspace supplies the workspace's device address
// (its status is returned if not PA_OK). Defined in pa_api.cpp.
int decode_with_library_workspace(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, float scale,
                                  int q_dtype, int cache_dtype, int out_dtype,
                                  const float* k_scale, const float* v_scale, int partition_tokens,
                                  int variant, int flags, size_t workspace_bytes,
                                  int (*resolve_workspace)(void**), void* stream);

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* tables, const int32_t* lens, int num_seqs,
                            int num_kv_heads, int head_dim, int block_size, int max_blocks,
                            int num_blocks, int max_tokens, int cache_dt, hipStream_t st);

}  // namespace pa
