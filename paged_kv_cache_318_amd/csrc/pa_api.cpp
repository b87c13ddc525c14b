// libpagedattn host side: the extern "C" entry points declared in include/pa.h.
//
// Every scalar argument is validated here before any HIP call, so a bad call returns an error
// code without touching the device; then the call picks a kernel variant and enqueues it on the
// caller's stream. The library allocates no device memory.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "pa.h"
#include "pa_launch.h"
#include "pa_sched.h"

namespace {

// Default partition lengths (tokens), from sweeps of 128..8192 on the decode workloads. The
// VALU kernel (one query head per work-group) is best at 512 on the partition-major grid, and over
// the ordered work list at 2048 once the batch has 2048 (sequence, query head) units or more (64
// sequences of 128..2048 tokens, 40 heads: 253.2 us with no merge launch, against 255.5 us + the
// merge at 512 partition-major; ordered 512 took 261.1 us, its many work-groups each paying the
// ordering's scans). The MFMA kernel (a whole query
// group per work-group: fewer, heavier work-groups, each paying a few microseconds to fetch its
// length, table entries and first tiles) is best at 1024 when there are many (sequence, kv head)
// units to spread over the CUs, and at 2048 when there are few (long sequences, split more).
// Over the ordered work list (longest work first, pa_sched.h) the MFMA kernel is best at 1024
// for 256..1023 units and at 2048 from 1024 units up (log-normal lengths, median 1024: 32, 64 and
// 128 sequences of 8 kv heads took 45.8, 76.3 and 145.7 us, against 48.1, 81.5 and 150.1 us for
// the partition-major grid at its best length, 1024).
// With few units the MFMA kernel instead takes the balanced split (one resident grid, each
// work-group a share of the tiles weighted by its order of arrival on its CU): on 16 sequences of
// 16K..32K tokens it takes 135 us, against 141 us for ordered 2048-token partitions, while on 128
// sequences of 64..8192 tokens (1024 units) the ordered partitions stay faster (146 us against
// 159 us), since there a work-group walks several short units, each starting with a table fetch
// and a first load round trip with nothing in flight.
// The ordered list is used from 1024-token partitions up, and not when sequences share blocks
// (PA_DECODE_SHARED_BLOCKS): there the partition-major grid keeps the samples of a prompt, whose
// shared blocks one fetch serves through the L2, running together (shared-prefix batch, 512-token
// partitions: 99.2 us against 104.7 us ordered).
// Workspaces are sized for the largest of these plans, so they fit every choice.
constexpr int kDefaultPartitionValu = 512;
constexpr int kDefaultPartitionValuOrdered = 2048;
constexpr int kManyValuUnitsOrdered = 2048;
constexpr int kMinOrderedPartition = 1024;
constexpr int kDefaultPartitionMfma = 1024;
constexpr int kDefaultPartitionMfmaFewUnits = 2048;
constexpr int kFewUnits = 256;
constexpr int kManyUnitsOrdered = 1024;
constexpr int kDefaultPartitionMfmaOrderedMany = 2048;
constexpr int kMaxGridYZ = 65535;
// HIP bounds gridDim.x * blockDim.x by 2^32 - 1 work-items: at most this many work-groups of 256
// threads (the widest block any kernel here launches) along x.
constexpr int64_t kMaxGridX = int64_t{0xFFFFFFFF} / 256;

bool dtype_ok(int dt) { return dt >= PA_F32 && dt <= PA_FP8_E4M3; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool block_size_ok(int b) { return b == 8 || b == 16 || b == 32; }

// ---- profiling (process-global; events recorded around launches when enabled) -------------------
struct EventPair {
  hipEvent_t start, stop;
};
constexpr int kKinds = PA_KERNEL_PREFILL + 1;
struct Profiler {
  bool on = false;
  std::vector<EventPair> pending[kKinds];
  std::vector<EventPair> pool;
  double ms[kKinds] = {};
  long long count[kKinds] = {};
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// Every timed pa_* call launches exactly one kernel: its event pair goes to that launch, which
// has the runtime stamp the kernel's own start and end (not the enqueue of a marker beside it).
bool begin_event(hipStream_t, EventPair* ev) {
  Profiler& P = prof();
  if (!P.on) return false;
  if (!P.pool.empty()) {
    *ev = P.pool.back();
    P.pool.pop_back();
  } else {
    if (hipEventCreate(&ev->start) != hipSuccess) return false;
    if (hipEventCreate(&ev->stop) != hipSuccess) {
      (void)hipEventDestroy(ev->start);
      return false;
    }
  }
  pa::dispatch_events() = pa::DispatchEvents{ev->start, ev->stop};
  return true;
}

void end_event(bool active, hipStream_t, const EventPair& ev, int kind) {
  if (!active) return;
  pa::DispatchEvents& pending = pa::dispatch_events();
  if (pending.start == nullptr) {
    prof().pending[kind].push_back(ev);  // the launch took the pair
  } else {
    pending = pa::DispatchEvents{};  // nothing was launched: the pair goes back unused
    prof().pool.push_back(ev);
  }
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Pointer kinds, from the runtime's own records. A pointer the runtime does not know (pageable
// host memory, a stale address) makes hipPointerGetAttributes fail; that error is cleared so it
// cannot surface at a later call.
bool pointer_kind(const void* p, hipPointerAttribute_t* attr) {
  if (hipPointerGetAttributes(attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

bool is_device_memory(const void* p) {
  hipPointerAttribute_t attr;
  return pointer_kind(p, &attr) && attr.type == hipMemoryTypeDevice;
}

// Pinned host memory: its address for kernels of the current device.
bool pinned_device_address(void* p, void** dev) {
  hipPointerAttribute_t attr;
  if (!pointer_kind(p, &attr) || attr.type != hipMemoryTypeHost) return false;
  if (hipHostGetDevicePointer(dev, p, 0) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return *dev != nullptr;
}
bool pinned_device_address(const void* p, void** dev) {
  return pinned_device_address(const_cast<void*>(p), dev);
}

// Partition plan shared by workspace sizing and the launch.
struct Plan {
  int part_blocks;
  int max_parts;
};
// units: (sequence, kv head) units for the MFMA kernel, (sequence, query head) for the VALU kernel;
// ordered: the batch may run over the ordered work list.
Plan plan_partitions(int max_blocks_per_seq, int block_size, int partition_tokens,
                     bool mfma = false, long long units = 0, bool ordered = false) {
  int pt = partition_tokens;
  if (pt <= 0) {
    if (!mfma)
      pt = ordered && units >= kManyValuUnitsOrdered ? kDefaultPartitionValuOrdered : kDefaultPartitionValu;
    else
      pt = units < kFewUnits ? kDefaultPartitionMfmaFewUnits
                             : (ordered && units >= kManyUnitsOrdered ? kDefaultPartitionMfmaOrderedMany
                                                                      : kDefaultPartitionMfma);
  }
  int pb = pt / block_size;
  if (pb < 1) pb = 1;
  return Plan{pb, (max_blocks_per_seq + pb - 1) / pb};
}

// Workspace of `slots` partial-result slots of `gu` heads each: normalised outputs [slots][gu][D]
// (fp32) followed by (max, sum) pairs [slots][gu].
size_t slot_bytes(size_t slots, int gu, int head_dim) {
  return slots * gu * (static_cast<size_t>(head_dim) * sizeof(float) + 2 * sizeof(float));
}

// Fixed partitions: one slot per (unit, partition), S * Hq * max_parts heads in all.
size_t fixed_workspace(int num_seqs, int num_heads, int head_dim, const Plan& pl) {
  if (pl.max_parts <= 1) return 0;
  return slot_bytes(static_cast<size_t>(num_seqs) * num_heads * pl.max_parts, 1, head_dim);
}

// The balanced split: for batches of few (sequence, kv head) units (the partition defaults above
// say why); it also needs the batch's lengths and block prefix sums in LDS and 32-bit block totals.
bool balanced_eligible(int num_seqs, int num_kv_heads, int max_blocks_per_seq) {
  return static_cast<long long>(num_seqs) * num_kv_heads < kFewUnits &&
         num_seqs <= pa::kMaxBalancedSeqs &&
         static_cast<int64_t>(num_seqs) * max_blocks_per_seq < (int64_t{1} << 31);
}

// CUs of the current device (cached per device; 0 if the runtime cannot tell).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape or dtype combination not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
    default: return "unknown pa_status";
  }
}

int pa_version(void) { return 100; }

int pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                int block_size, int num_blocks, pa_dtype in_dtype, pa_dtype cache_dtype,
                const float* k_scale, const float* v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(cache_dtype)) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (in_dtype == PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (cache_dtype != PA_FP8_E4M3 && cache_dtype != in_dtype) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(num_tokens) + block_size - 1) / block_size > kMaxGridX)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  const bool timed = begin_event(st, &ev);
  const hipError_t e = pa::launch_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping,
                                           num_tokens, num_kv_heads, head_dim, block_size,
                                           num_blocks, in_dtype, cache_dtype, k_scale, v_scale, st);
  end_event(timed, st, ev, PA_KERNEL_WRITE_KV);
  return hip_status(e);
}

int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, pa_dtype cache_dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (!dtype_ok(cache_dtype)) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (num_pairs > kMaxGridX) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_INVALID_ARG;
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  const bool timed = begin_event(st, &ev);
  const hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, k_scale, v_scale, block_pairs,
                                              num_pairs, num_kv_heads, head_dim, block_size,
                                              num_blocks, cache_dtype, st);
  end_event(timed, st, ev, PA_KERNEL_COPY_BLOCKS);
  return hip_status(e);
}

int pa_swap_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int num_blocks,
                   void* host_k, void* host_v, float* host_k_scale, float* host_v_scale,
                   int num_host_blocks, const int32_t* block_pairs, int num_pairs, int direction,
                   int num_kv_heads, int head_dim, int block_size, pa_dtype cache_dtype,
                   void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0 || num_host_blocks <= 0 ||
      head_dim <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN) return PA_ERR_INVALID_ARG;
  if (!dtype_ok(cache_dtype)) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (num_pairs > kMaxGridX) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  if (!k_cache || !v_cache || !host_k || !host_v || !block_pairs) return PA_ERR_INVALID_ARG;
  if (fp8 && (!k_scale || !v_scale || !host_k_scale || !host_v_scale)) return PA_ERR_INVALID_ARG;
  // Device-side addresses of the pinned host pool; nothing is launched unless every pointer is of
  // the kind the kernel can access.
  void* dk = nullptr;
  void* dv = nullptr;
  void* dks = nullptr;
  void* dvs = nullptr;
  if (!is_device_memory(k_cache) || !is_device_memory(v_cache) ||
      (fp8 && (!is_device_memory(k_scale) || !is_device_memory(v_scale))))
    return PA_ERR_INVALID_ARG;
  if (!pinned_device_address(host_k, &dk) || !pinned_device_address(host_v, &dv) ||
      (fp8 && (!pinned_device_address(host_k_scale, &dks) ||
               !pinned_device_address(host_v_scale, &dvs))))
    return PA_ERR_INVALID_ARG;
  const void* pairs = block_pairs;
  if (!is_device_memory(block_pairs)) {
    void* dp = nullptr;
    if (!pinned_device_address(block_pairs, &dp)) return PA_ERR_INVALID_ARG;
    pairs = dp;
  }
  const bool out = direction == PA_SWAP_OUT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  const bool timed = begin_event(st, &ev);
  const hipError_t e =
      out ? pa::launch_swap_blocks(k_cache, v_cache, dk, dv, k_scale, v_scale,
                                   static_cast<float*>(dks), static_cast<float*>(dvs),
                                   static_cast<const int32_t*>(pairs), num_pairs, num_blocks,
                                   num_host_blocks, num_kv_heads, head_dim, block_size,
                                   cache_dtype, st)
          : pa::launch_swap_blocks(dk, dv, k_cache, v_cache, static_cast<const float*>(dks),
                                   static_cast<const float*>(dvs), k_scale, v_scale,
                                   static_cast<const int32_t*>(pairs), num_pairs, num_host_blocks,
                                   num_blocks, num_kv_heads, head_dim, block_size, cache_dtype,
                                   st);
  end_event(timed, st, ev, PA_KERNEL_SWAP_BLOCKS);
  return hip_status(e);
}

int pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                 int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                 int num_blocks, int max_tokens, pa_dtype cache_dtype, void* stream) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || max_tokens <= 0)
    return PA_ERR_INVALID_ARG;
  if (!dtype_ok(cache_dtype)) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (max_tokens > max_blocks_per_seq * block_size) return PA_ERR_INVALID_ARG;
  if (num_seqs > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(max_tokens) + block_size - 1) / block_size > kMaxGridX)
    return PA_ERR_UNSUPPORTED;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  const bool timed = begin_event(st, &ev);
  const hipError_t e = pa::launch_gather_kv(k_out, v_out, k_cache, v_cache, block_tables,
                                            context_lens, num_seqs, num_kv_heads, head_dim,
                                            block_size, max_blocks_per_seq, num_blocks,
                                            max_tokens, cache_dtype, st);
  end_event(timed, st, ev, PA_KERNEL_GATHER_KV);
  return hip_status(e);
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int block_size, int partition_tokens) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      head_dim <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 || partition_tokens < 0)
    return 0;
  if (partition_tokens > 0)
    return fixed_workspace(num_seqs, num_heads, head_dim,
                           plan_partitions(max_blocks_per_seq, block_size, partition_tokens));
  // default plan: fixed partitions of the shortest default length, or the balanced split
  size_t need = fixed_workspace(num_seqs, num_heads, head_dim,
                                plan_partitions(max_blocks_per_seq, block_size, 0));
  if (balanced_eligible(num_seqs, num_kv_heads, max_blocks_per_seq)) {
    const int G = num_heads / num_kv_heads;
    const size_t bal = slot_bytes(2 * static_cast<size_t>(pa::kMaxBalancedGroups), G <= 16 ? G : 1, head_dim) +
                       (pa::kMaxBalancedSeqs + 1) * sizeof(int);
    need = need > bal ? need : bal;
  }
  return need;
}

namespace {

// Checks shared by pa_decode, pa_decode_append and pa_decode_grouped: sizes, scale, dtypes,
// flags, partition length, 32-bit slot ranges, supported shapes and dtype pairs, pointers.
int check_decode_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
                      pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
                      const float* v_scale, int partition_tokens, int flags) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!dtype_ok(q_dtype) || !dtype_ok(cache_dtype) || !dtype_ok(out_dtype)) return PA_ERR_INVALID_ARG;
  if ((flags & ~PA_DECODE_SHARED_BLOCKS) != 0) return PA_ERR_INVALID_ARG;
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % block_size != 0))
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const bool pair_ok = (cache_dtype == q_dtype && q_dtype != PA_FP8_E4M3) ||
                       (cache_dtype == PA_FP8_E4M3 && (q_dtype == PA_F16 || q_dtype == PA_BF16));
  if (!pair_ok) return PA_ERR_UNSUPPORTED;
  if (out_dtype != q_dtype && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// pa_decode, and pa_decode_append when k_new != nullptr (new tokens taken along and written).
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                int num_heads, int num_kv_heads, int head_dim, int block_size,
                int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
                pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
                const float* v_scale, int partition_tokens, int variant, int flags,
                void* workspace, size_t workspace_bytes, void* stream, const void* k_new,
                const void* v_new, const int32_t* slot_mapping,
                int (*resolve_workspace)(void**) = nullptr) {
  if (variant < PA_VARIANT_AUTO || variant > PA_VARIANT_MFMA) return PA_ERR_INVALID_ARG;
  const int status = check_decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                       num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype,
                                       out_dtype, k_scale, v_scale, partition_tokens, flags);
  if (status != PA_OK) return status;
  const int G = num_heads / num_kv_heads;
  const bool mfma_ok = cache_dtype != PA_F32 && G <= 16;  // block sizes 8, 16 and 32
  bool use_mfma;
  if (variant == PA_VARIANT_MFMA) {
    if (!mfma_ok) return PA_ERR_UNSUPPORTED;
    use_mfma = true;
  } else if (variant == PA_VARIANT_VALU) {
    use_mfma = false;
  } else {
    use_mfma = mfma_ok && G >= 2;
  }
  const long long units = static_cast<long long>(num_seqs) * (use_mfma ? num_kv_heads : num_heads);
  const bool stream_kv = (flags & PA_DECODE_SHARED_BLOCKS) == 0;
  // Default plan for the MFMA kernel on few units: the balanced split over one resident grid.
  const bool balanced =
      partition_tokens == 0 && use_mfma && balanced_eligible(num_seqs, num_kv_heads, max_blocks_per_seq);
  // Fixed partitions may run over the ordered work list (longest work first) when the batch's
  // lengths fit the ordering's LDS. The partition length does not depend on the shared-blocks
  // flag, which only selects the cache policy and the grid order: the same inputs give the same
  // bits with or without it.
  const bool order_ok = !balanced && num_seqs <= pa::kOrderedMaxSeqs;
  const Plan pl = plan_partitions(max_blocks_per_seq, block_size, partition_tokens, use_mfma, units,
                                  order_ok);
  if (num_seqs > kMaxGridYZ || pl.max_parts > kMaxGridYZ || num_heads > kMaxGridX)
    return PA_ERR_UNSUPPORTED;
  int nw = 0, nw_cls = 0;
  if (balanced) {
    const int per_cu = pa::mfma_groups_per_cu(cache_dtype, q_dtype, head_dim, block_size, G, num_seqs);
    const int cus = cu_count();
    nw = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
    nw = nw > pa::kMaxBalancedGroups ? pa::kMaxBalancedGroups : nw;
    // three resident work-groups per CU: shares weighted by their order of arrival on the CU
    if (cus > 0 && per_cu == 3 && nw == 3 * cus) nw_cls = cus;
  }
  const int gu = use_mfma ? G : 1;
  const size_t slots = balanced ? 2 * static_cast<size_t>(nw)
                                : static_cast<size_t>(num_seqs) * (num_heads / gu) * pl.max_parts;
  const size_t need = balanced ? slot_bytes(slots, gu, head_dim) + (num_seqs + 1) * sizeof(int)
                               : fixed_workspace(num_seqs, num_heads, head_dim, pl);
  if (need > 0 && workspace_bytes < need) return PA_ERR_WORKSPACE;
  // a workspace the library provides itself is looked up only now, after every host check
  if (need > 0 && workspace == nullptr && resolve_workspace != nullptr) {
    const int ws_status = resolve_workspace(&workspace);
    if (ws_status != PA_OK) return ws_status;
  }
  if (need > 0 && workspace == nullptr) return PA_ERR_WORKSPACE;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.tables = block_tables;
  a.lens = context_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.ws_o = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need > 0 ? reinterpret_cast<float2*>(static_cast<uint8_t*>(workspace) +
                                                 slots * gu * head_dim * sizeof(float))
                     : nullptr;
  a.ws_pref = balanced ? reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) +
                                                slot_bytes(slots, gu, head_dim))
                       : nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.part_blocks = pl.part_blocks;
  a.max_parts = pl.max_parts;
  a.out_dtype = out_dtype;
  a.zscale = scale * pa::kLog2e;
  a.stream_kv = stream_kv ? 1 : 0;
  a.heads_per_unit = gu;
  a.balanced = balanced ? 1 : 0;
  a.nw = nw;
  a.nw_cls = nw_cls;
  // (the ordered list's 1-D grid must also fit, else the 3-D grid takes the batch; the
  // ordering's length classes multiply a partition's block count by 16 in 32 bits)
  a.ordered = (order_ok && stream_kv && static_cast<int64_t>(pl.part_blocks) * block_size >= kMinOrderedPartition &&
               pl.part_blocks <= (1 << 26) && pa::xcd_weighted_grid(units * pl.max_parts) <= kMaxGridX) ? 1 : 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = k_new != nullptr ? slot_mapping : nullptr;

  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  bool timed = begin_event(st, &ev);
  hipError_t e = use_mfma ? pa::launch_decode_mfma(a, cache_dtype, q_dtype, head_dim, block_size, st)
                          : pa::launch_decode_valu(a, cache_dtype, q_dtype, head_dim, block_size, st);
  end_event(timed, st, ev, PA_KERNEL_DECODE_PARTITION);
  if (e != hipSuccess) return PA_ERR_HIP;
  if (balanced || pl.max_parts > 1) {
    timed = begin_event(st, &ev);
    e = pa::launch_decode_merge(a, head_dim, block_size, st);
    end_event(timed, st, ev, PA_KERNEL_DECODE_MERGE);
  }
  return hip_status(e);
}

}  // namespace

namespace {

// Grouped decode plan: MFMA partitions (of the default length for many units, or the caller's),
// one more part per (sequence, head) for the split between prefix and own blocks.
Plan grouped_plan(int max_blocks_per_seq, int block_size, int partition_tokens) {
  Plan pl = plan_partitions(max_blocks_per_seq, block_size, partition_tokens, true, kFewUnits);
  pl.max_parts += 1;
  return pl;
}

size_t grouped_workspace(int num_seqs, int num_heads, int head_dim, const Plan& pl) {
  return slot_bytes(static_cast<size_t>(num_seqs) * num_heads * pl.max_parts, 1, head_dim) +
         static_cast<size_t>(num_seqs) * sizeof(int);
}

}  // namespace

size_t pa_decode_grouped_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                         int max_blocks_per_seq, int block_size,
                                         int partition_tokens) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0 || partition_tokens < 0)
    return 0;
  return grouped_workspace(num_seqs, num_heads, head_dim,
                           grouped_plan(max_blocks_per_seq, block_size, partition_tokens));
}

// pa_decode_grouped, and pa_decode_grouped_append when k_new != nullptr (new tokens taken along
// and written by the work-group holding each sequence's last block).
static int grouped_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* group_start, const int32_t* prefix_blocks, int num_groups,
                        int max_group_size, int num_seqs, int num_heads, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                        float scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                        const float* k_scale, const float* v_scale, int partition_tokens, int flags,
                        void* workspace, size_t workspace_bytes, void* stream, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping) {
  if (num_groups <= 0 || max_group_size <= 0 || num_groups > num_seqs) return PA_ERR_INVALID_ARG;
  const int status = check_decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                       num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, num_blocks, scale, q_dtype, cache_dtype,
                                       out_dtype, k_scale, v_scale, partition_tokens, flags);
  if (status != PA_OK) return status;
  if (cache_dtype == PA_F32) return PA_ERR_UNSUPPORTED;  // the matrix-core kernel only
  const int G = num_heads / num_kv_heads;
  if (static_cast<int64_t>(max_group_size) * G > 16) return PA_ERR_UNSUPPORTED;
  if (!group_start || !prefix_blocks) return PA_ERR_INVALID_ARG;
  const Plan pl = grouped_plan(max_blocks_per_seq, block_size, partition_tokens);
  if (static_cast<int64_t>(num_seqs) + num_groups > kMaxGridYZ || pl.max_parts > kMaxGridYZ ||
      num_heads > kMaxGridX)
    return PA_ERR_UNSUPPORTED;
  const size_t need = grouped_workspace(num_seqs, num_heads, head_dim, pl);
  if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const size_t slots = static_cast<size_t>(num_seqs) * num_heads * pl.max_parts;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.tables = block_tables;
  a.lens = context_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float2*>(static_cast<uint8_t*>(workspace) + slots * head_dim * sizeof(float));
  a.ws_count = reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) + slot_bytes(slots, 1, head_dim));
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.part_blocks = pl.part_blocks;
  a.max_parts = pl.max_parts;
  a.out_dtype = out_dtype;
  a.zscale = scale * pa::kLog2e;
  a.stream_kv = (flags & PA_DECODE_SHARED_BLOCKS) == 0 ? 1 : 0;
  a.heads_per_unit = 1;
  a.grouped = 1;
  a.num_groups = num_groups;
  a.group_start = group_start;
  a.prefix_blocks = prefix_blocks;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = k_new != nullptr ? slot_mapping : nullptr;

  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  bool timed = begin_event(st, &ev);
  hipError_t e = pa::launch_decode_mfma(a, cache_dtype, q_dtype, head_dim, block_size, st);
  end_event(timed, st, ev, PA_KERNEL_DECODE_PARTITION);
  if (e != hipSuccess) return PA_ERR_HIP;
  timed = begin_event(st, &ev);
  e = pa::launch_decode_merge(a, head_dim, block_size, st);
  end_event(timed, st, ev, PA_KERNEL_DECODE_MERGE);
  return hip_status(e);
}

int pa_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* group_start, const int32_t* prefix_blocks, int num_groups,
                      int max_group_size, int num_seqs, int num_heads, int num_kv_heads,
                      int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                      float scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                      const float* k_scale, const float* v_scale, int partition_tokens, int flags,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_impl(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                      prefix_blocks, num_groups, max_group_size, num_seqs, num_heads, num_kv_heads,
                      head_dim, block_size, max_blocks_per_seq, num_blocks, scale, q_dtype,
                      cache_dtype, out_dtype, k_scale, v_scale, partition_tokens, flags, workspace,
                      workspace_bytes, stream, nullptr, nullptr, nullptr);
}

int pa_decode_grouped_append(void* out, const void* q, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const void* k_new, const void* v_new, const int32_t* slot_mapping,
                             pa_dtype new_dtype, const int32_t* group_start,
                             const int32_t* prefix_blocks, int num_groups, int max_group_size,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                             pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                             const float* k_scale, const float* v_scale, int partition_tokens,
                             int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(new_dtype) || !dtype_ok(cache_dtype) || !dtype_ok(q_dtype)) return PA_ERR_INVALID_ARG;
  // the new rows are stored as they are (16-bit caches) or quantised from the query type (fp8)
  if (new_dtype != (cache_dtype == PA_FP8_E4M3 ? q_dtype : cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return grouped_impl(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                      prefix_blocks, num_groups, max_group_size, num_seqs, num_heads, num_kv_heads,
                      head_dim, block_size, max_blocks_per_seq, num_blocks, scale, q_dtype,
                      cache_dtype, out_dtype, k_scale, v_scale, partition_tokens, flags, workspace,
                      workspace_bytes, stream, k_new, v_new, slot_mapping);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
              pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
              const float* v_scale, int partition_tokens, int variant, int flags,
              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     q_dtype, cache_dtype, out_dtype, k_scale, v_scale, partition_tokens, variant,
                     flags, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

int pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, const void* k_new,
                     const void* v_new, const int32_t* slot_mapping, pa_dtype new_dtype,
                     int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int num_blocks, float scale, pa_dtype q_dtype,
                     pa_dtype cache_dtype, pa_dtype out_dtype, const float* k_scale,
                     const float* v_scale, int partition_tokens, int variant, int flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(new_dtype) || !dtype_ok(cache_dtype) || !dtype_ok(q_dtype)) return PA_ERR_INVALID_ARG;
  // the new rows are stored as they are (16/32-bit caches) or quantised from the query type (fp8)
  if (new_dtype != (cache_dtype == PA_FP8_E4M3 ? q_dtype : cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     q_dtype, cache_dtype, out_dtype, k_scale, v_scale, partition_tokens, variant,
                     flags, workspace, workspace_bytes, stream, k_new, v_new, slot_mapping);
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
               int num_seqs, int num_tokens, int max_query_len, int num_heads, int num_kv_heads,
               int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
               pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
               const float* k_scale, const float* v_scale, void* stream) {
  if (num_seqs <= 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!dtype_ok(q_dtype) || !dtype_ok(cache_dtype) || !dtype_ok(out_dtype)) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_blocks) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size >= (int64_t{1} << 31)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (max_query_len <= 0) return PA_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const bool pair_ok = ((cache_dtype == PA_F16 || cache_dtype == PA_BF16) && q_dtype == cache_dtype) ||
                       (cache_dtype == PA_FP8_E4M3 && (q_dtype == PA_F16 || q_dtype == PA_BF16));
  if (!pair_ok) return PA_ERR_UNSUPPORTED;
  if (out_dtype != q_dtype && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  // one work-group per (64-row tile, kv head, sequence), in a one-dimensional grid
  if ((static_cast<int64_t>(max_query_len) * G + 63) / 64 * num_kv_heads * num_seqs > kMaxGridX)
    return PA_ERR_UNSUPPORTED;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_INVALID_ARG;
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.tables = block_tables;
  a.lens = context_lens;
  a.query_start = query_start;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.out_dtype = out_dtype;
  a.zscale = scale * pa::kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPair ev;
  const bool timed = begin_event(st, &ev);
  const hipError_t e = pa::launch_prefill(a, cache_dtype, q_dtype, head_dim, block_size, max_query_len, st);
  end_event(timed, st, ev, PA_KERNEL_PREFILL);
  return hip_status(e);
}

int pa_profile_enable(int on) {
  Profiler& P = prof();
  for (int k = 0; k < kKinds; ++k) {
    for (const EventPair& ev : P.pending[k]) P.pool.push_back(ev);
    P.pending[k].clear();
    P.ms[k] = 0.0;
    P.count[k] = 0;
  }
  P.on = on != 0;
  return PA_OK;
}

int pa_profile_read(int kernel_kind, double* total_ms, long long* launches) {
  if (kernel_kind < 0 || kernel_kind >= kKinds || !total_ms || !launches) return PA_ERR_INVALID_ARG;
  Profiler& P = prof();
  for (const EventPair& ev : P.pending[kernel_kind]) {
    if (hipEventSynchronize(ev.stop) != hipSuccess) return PA_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, ev.start, ev.stop) != hipSuccess) return PA_ERR_HIP;
    P.ms[kernel_kind] += ms;
    P.count[kernel_kind] += 1;
    P.pool.push_back(ev);
  }
  P.pending[kernel_kind].clear();
  *total_ms = P.ms[kernel_kind];
  *launches = P.count[kernel_kind];
  return PA_OK;
}

}  // extern "C"

// Not an entry point of the ABI: the allocation-free decode (decode_noalloc.hip) reaches pa_decode's
// host logic through here.
namespace pa {

DispatchEvents& dispatch_events() {
  thread_local DispatchEvents pending;
  return pending;
}

int decode_with_library_workspace(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, float scale,
                                  int q_dtype, int cache_dtype, int out_dtype,
                                  const float* k_scale, const float* v_scale, int partition_tokens,
                                  int variant, int flags, size_t workspace_bytes,
                                  int (*resolve_workspace)(void**), void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     static_cast<pa_dtype>(q_dtype), static_cast<pa_dtype>(cache_dtype),
                     static_cast<pa_dtype>(out_dtype), k_scale, v_scale, partition_tokens, variant,
                     flags, nullptr, workspace_bytes, stream, nullptr, nullptr, nullptr,
                     resolve_workspace);
}

}  // namespace pa
