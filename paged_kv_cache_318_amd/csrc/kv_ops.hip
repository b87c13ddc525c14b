// KV-cache moves on gfx950: slot-mapped write of new tokens, whole-block copy for
// copy-on-write, and read-back of sequences through their block tables.
//
// "PagedAttention", Ultralytics glossary: section "ページングの仕組み" (how paging works) --
// a token at position pos goes to slot pos mod B of the block the table lists at index pos div B,
// and a request is read back through its table; section "シーケンス間でのブロック共有" (sharing
// blocks between sequences) -- a block still used by another sequence is copied before a write.
//
// Layouts: k_cache [NB][Hkv][B][D] (a token's key is a contiguous row of D elements),
// v_cache [NB][Hkv][D][B] (values are dim-major inside a block), fp8 scales [NB][Hkv].

#include "kv_write.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {


// One work-group per (group of B consecutive new tokens, kv head). When the group's slots are one
// whole block in order -- the common case of a prompt or a chunk -- the values are transposed
// through LDS and every dim row of the block's value tile is written whole (B * elem bytes,
// 16-byte stores) instead of one element per row and token; any other group (decode tokens of
// different sequences, the partial first and last block of a chunk, skipped tokens) writes piece
// by piece. Keys are token rows either way. grid = (ceil(num_tokens / B), Hkv).
template <int IN_DT, int C_DT>
__global__ __launch_bounds__(256) void write_kv_kernel(const void* __restrict__ k_new,
                                                       const void* __restrict__ v_new,
                                                       void* __restrict__ k_cache,
                                                       void* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slots, int T,
                                                       int Hkv, int D, int B, int NB,
                                                       const float* __restrict__ k_scale,
                                                       const float* __restrict__ v_scale) {
  constexpr int IEB = Elem<IN_DT>::bytes;
  constexpr int CEB = Elem<C_DT>::bytes;
  using CT = typename Store<C_DT>::T;
  __shared__ int s_slot[32];
  __shared__ __align__(16) uint8_t tile[128 * 32 * 4];  // [D][B] values of one block, cache type
  const int t0 = blockIdx.x * B, hh = blockIdx.y, tid = threadIdx.x;
  const int nt = T - t0 < B ? T - t0 : B;
  if (tid < B) {
    int sl = tid < nt ? slots[t0 + tid] : -1;
    s_slot[tid] = (sl < 0 || sl >= NB * B) ? -1 : sl;  // skipped (or out-of-range: ignored)
  }
  __syncthreads();
  // whole block in order: B valid slots, the first at a block boundary, each the next
  const int base = s_slot[0];
  const bool in_order = tid >= B || (nt == B && base >= 0 && base % B == 0 && s_slot[tid] == base + tid);
  const bool whole = __syncthreads_and(in_order) != 0;
  const int per_tok = D / 8;                 // 8-dim pieces of one token's head
  if (!whole) {
    for (int w = tid; w < nt * per_tok; w += blockDim.x) {
      const int i = w / per_tok, d0 = (w - i * per_tok) * 8;
      const int sl = s_slot[i];
      if (sl < 0) continue;
      write_piece<IN_DT, C_DT, true>(k_new, v_new, k_cache, v_cache, t0 + i, sl, hh, d0, Hkv, D, B,
                                     k_scale, v_scale);
    }
    return;
  }
  // keys are token rows; values of the whole block go through LDS: token i's 8 dims d0.. land in
  // column i of rows d0..d0+7. Each piece's value load is issued before its key load, so both
  // are in flight together.
  const int b = base / B;
  CT* tl = reinterpret_cast<CT*>(tile);
  float vs = 1.0f;
  if constexpr (C_DT == DT_FP8) vs = v_scale[static_cast<size_t>(b) * Hkv + hh];
  for (int w = tid; w < B * per_tok; w += blockDim.x) {
    const int i = w / per_tok, d0 = (w - i * per_tok) * 8;
    const size_t src = (static_cast<size_t>(t0 + i) * Hkv + hh) * D + d0;
    const Raw<8 * IEB> vr = load_raw<8 * IEB>(reinterpret_cast<const uint8_t*>(v_new) + src * IEB);
    write_piece<IN_DT, C_DT, false>(k_new, v_new, k_cache, v_cache, t0 + i, base + i, hh, d0, Hkv, D,
                                    B, k_scale, v_scale);
    if constexpr (C_DT == DT_FP8) {
      float vf[8];
      to_f32<IN_DT, 8>(vr.w, vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) tl[(d0 + e) * B + i] = static_cast<CT>(f32_to_e4m3(vf[e] / vs, vf[e]));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        CT v;
        if constexpr (CEB == 4) v = vr.w[e];
        else v = static_cast<CT>(vr.w[e / 2] >> (16 * (e & 1)));
        tl[(d0 + e) * B + i] = v;
      }
    }
  }
  __syncthreads();
  // the tile is the block's [D][B] value slab for this head: contiguous in the cache
  const int n16 = D * B * CEB / 16;
  u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(v_cache) +
                                        (static_cast<size_t>(b) * Hkv + hh) * D * B * CEB);
  const u32x4* srcl = reinterpret_cast<const u32x4*>(tile);
  for (int w = tid; w < n16; w += blockDim.x) dst[w] = srcl[w];
}

// grid.x = pair, grid.y = chunk of the block; 16-byte copies of both caches from block src of
// the source pool to block dst of the destination pool (one pool for copy-on-write, so the two may
// alias; the device pool and a pinned host pool for swaps). Pairs naming a block outside either
// pool are skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(const uint8_t* src_k, const uint8_t* src_v,
                                                          uint8_t* dst_k, uint8_t* dst_v,
                                                          const float* src_ks, const float* src_vs,
                                                          float* dst_ks, float* dst_vs,
                                                          const int32_t* pairs, int src_nb,
                                                          int dst_nb, int Hkv, size_t block_bytes) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_nb || dst < 0 || dst >= dst_nb) return;
  const size_t n16 = block_bytes / 16;
  const u32x4* ks = reinterpret_cast<const u32x4*>(src_k + static_cast<size_t>(src) * block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(src_v + static_cast<size_t>(src) * block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(dst_k + static_cast<size_t>(dst) * block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(dst_v + static_cast<size_t>(dst) * block_bytes);
  for (size_t i = static_cast<size_t>(blockIdx.y) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.y) * blockDim.x) {
    const u32x4 a = ks[i];
    const u32x4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
  if (src_ks != nullptr && blockIdx.y == 0) {
    for (int hh = threadIdx.x; hh < Hkv; hh += blockDim.x) {
      dst_ks[static_cast<size_t>(dst) * Hkv + hh] = src_ks[static_cast<size_t>(src) * Hkv + hh];
      dst_vs[static_cast<size_t>(dst) * Hkv + hh] = src_vs[static_cast<size_t>(src) * Hkv + hh];
    }
  }
}

// grid = (logical block j, sequence s); copies the block's valid tokens out in logical order.
template <typename T>
__global__ __launch_bounds__(256) void gather_kv_kernel(T* k_out, T* v_out, const T* k_cache,
                                                        const T* v_cache, const int32_t* tables,
                                                        const int32_t* lens, int Hkv, int D,
                                                        int B, int MB, int NB, int max_tokens) {
  const int j = blockIdx.x, s = blockIdx.y;
  int L = lens[s];
  L = L < 0 ? 0 : (L > MB * B ? MB * B : L);
  L = L < max_tokens ? L : max_tokens;
  const int t0 = j * B;
  if (t0 >= L) return;
  int pb = tables[static_cast<size_t>(s) * MB + j];
  pb = pb < 0 ? 0 : (pb >= NB ? NB - 1 : pb);
  const int nt = (L - t0) < B ? (L - t0) : B;
  const int n = nt * Hkv * D;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int o = idx / (Hkv * D);
    const int rem = idx - o * (Hkv * D);
    const int hh = rem / D, d = rem - (rem / D) * D;
    const size_t dst = (static_cast<size_t>(s) * max_tokens + t0 + o) * Hkv * D + rem;
    k_out[dst] = k_cache[((static_cast<size_t>(pb) * Hkv + hh) * B + o) * D + d];
    v_out[dst] = v_cache[((static_cast<size_t>(pb) * Hkv + hh) * D + d) * B + o];
  }
}

// ---- launchers ----------------------------------------------------------------------------------
hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* slots, int T, int Hkv, int D, int B, int NB, int in_dt,
                           int cache_dt, const float* k_scale, const float* v_scale,
                           hipStream_t st) {
  const dim3 grid((T + B - 1) / B, Hkv), block(256);
#define PA_WRITE(I, C)                                                                         \
  launch_kernel((write_kv_kernel<I, C>), grid, block, 0, st, k_new, v_new, k_cache,       \
                     v_cache, slots, T, Hkv, D, B, NB, k_scale, v_scale)
  if (cache_dt == DT_FP8) {
    if (in_dt == DT_F32) PA_WRITE(DT_F32, DT_FP8);
    else if (in_dt == DT_F16) PA_WRITE(DT_F16, DT_FP8);
    else if (in_dt == DT_BF16) PA_WRITE(DT_BF16, DT_FP8);
    else return hipErrorInvalidValue;
  } else if (cache_dt == in_dt) {
    if (in_dt == DT_F32) PA_WRITE(DT_F32, DT_F32);
    else if (in_dt == DT_F16) PA_WRITE(DT_F16, DT_F16);
    else if (in_dt == DT_BF16) PA_WRITE(DT_BF16, DT_BF16);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
#undef PA_WRITE
  return hipGetLastError();
}

// Chunks per block: about 8 16-byte copies per thread and cache, at most 64 work-groups a block.
static int copy_chunks(size_t block_bytes) {
  const size_t n16 = block_bytes / 16;
  const int chunks = static_cast<int>((n16 + 2047) / 2048);
  return chunks < 1 ? 1 : (chunks > 64 ? 64 : chunks);
}

static size_t block_bytes_of(int Hkv, int D, int B, int cache_dt) {
  const int eb = cache_dt == DT_F32 ? 4 : (cache_dt == DT_FP8 ? 1 : 2);
  return static_cast<size_t>(Hkv) * B * D * eb;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int num_pairs, int Hkv, int D, int B, int NB,
                              int cache_dt, hipStream_t st) {
  const size_t block_bytes = block_bytes_of(Hkv, D, B, cache_dt);
  const bool fp8 = cache_dt == DT_FP8;
  uint8_t* k = reinterpret_cast<uint8_t*>(k_cache);
  uint8_t* v = reinterpret_cast<uint8_t*>(v_cache);
  launch_kernel(copy_blocks_kernel, dim3(num_pairs, copy_chunks(block_bytes)), dim3(256), 0,
                     st, k, v, k, v, fp8 ? k_scale : nullptr, fp8 ? v_scale : nullptr,
                     fp8 ? k_scale : nullptr, fp8 ? v_scale : nullptr, pairs, NB, NB, Hkv,
                     block_bytes);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const float* src_ks, const float* src_vs, float* dst_ks,
                              float* dst_vs, const int32_t* pairs, int num_pairs, int src_nb,
                              int dst_nb, int Hkv, int D, int B, int cache_dt, hipStream_t st) {
  const size_t block_bytes = block_bytes_of(Hkv, D, B, cache_dt);
  const bool fp8 = cache_dt == DT_FP8;
  launch_kernel(copy_blocks_kernel, dim3(num_pairs, copy_chunks(block_bytes)), dim3(256), 0,
                     st, reinterpret_cast<const uint8_t*>(src_k),
                     reinterpret_cast<const uint8_t*>(src_v), reinterpret_cast<uint8_t*>(dst_k),
                     reinterpret_cast<uint8_t*>(dst_v), fp8 ? src_ks : nullptr,
                     fp8 ? src_vs : nullptr, fp8 ? dst_ks : nullptr, fp8 ? dst_vs : nullptr, pairs,
                     src_nb, dst_nb, Hkv, block_bytes);
  return hipGetLastError();
}

hipError_t launch_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* tables, const int32_t* lens, int S, int Hkv, int D,
                            int B, int MB, int NB, int max_tokens, int cache_dt, hipStream_t st) {
  const int mbt = (max_tokens + B - 1) / B;
  const dim3 grid(mbt < MB ? mbt : MB, S), block(256);
#define PA_GATHER(T)                                                                            \
  launch_kernel((gather_kv_kernel<T>), grid, block, 0, st, reinterpret_cast<T*>(k_out),    \
                     reinterpret_cast<T*>(v_out), reinterpret_cast<const T*>(k_cache),          \
                     reinterpret_cast<const T*>(v_cache), tables, lens, Hkv, D, B, MB, NB,     \
                     max_tokens)
  if (cache_dt == DT_F32) PA_GATHER(uint32_t);
  else if (cache_dt == DT_FP8) PA_GATHER(uint8_t);
  else PA_GATHER(uint16_t);
#undef PA_GATHER
  return hipGetLastError();
}

}  // namespace pa
