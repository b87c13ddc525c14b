// Device-side helpers shared by the gfx950 kernels of libpagedattn: element traits, raw vector
// loads, storage <-> fp32 conversions, DPP row reductions, and the argument blocks the host
// passes to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP8> { static constexpr int bytes = 1; };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// ---- raw loads of NB bytes (NB in {2, 4, 8, 16, 32, 64}); the address is NB-aligned (or
// 16-aligned for NB >= 16) by construction of the layouts -------------------------------------
template <int NB> struct Raw { uint32_t w[NB >= 4 ? NB / 4 : 1]; };

// NT = true marks the load non-temporal (streamed through the caches, allocated for eviction
// first): used for K/V tiles, which are read exactly once per call, when every load instruction
// of a wave covers whole 128-byte lines.
template <int NB, bool NT = false>
__device__ __forceinline__ Raw<NB> load_raw(const void* p) {
  Raw<NB> r;
  if constexpr (NB == 2) {
    r.w[0] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p))
                : *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (NB == 4) {
    r.w[0] = NT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p))
                : *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NB == 8) {
    u32x2 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                 : *reinterpret_cast<const u32x2*>(p);
    r.w[0] = v.x;
    r.w[1] = v.y;
  } else {
    static_assert(NB % 16 == 0, "unsupported load width");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      u32x4 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i)
                   : reinterpret_cast<const u32x4*>(p)[i];
      r.w[4 * i + 0] = v.x;
      r.w[4 * i + 1] = v.y;
      r.w[4 * i + 2] = v.z;
      r.w[4 * i + 3] = v.w;
    }
  }
  return r;
}

// Stores NB bytes (a Raw piece) at an NB-aligned address.
template <int NB>
__device__ __forceinline__ void store_raw(void* p, const Raw<NB>& r) {
  if constexpr (NB == 2) {
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(r.w[0]);
  } else if constexpr (NB == 4) {
    *reinterpret_cast<uint32_t*>(p) = r.w[0];
  } else if constexpr (NB == 8) {
    *reinterpret_cast<u32x2*>(p) = u32x2{r.w[0], r.w[1]};
  } else {
    static_assert(NB % 16 == 0, "unsupported store width");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      reinterpret_cast<u32x4*>(p)[i] = u32x4{r.w[4 * i], r.w[4 * i + 1], r.w[4 * i + 2], r.w[4 * i + 3]};
  }
}

// ---- storage -> fp32 (all exact) -------------------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xffffu)));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Converts N consecutive stored elements (packed little-endian in words w) to fp32.
template <int DT, int N>
__device__ __forceinline__ void to_f32(const uint32_t* w, float* f) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == DT_F16) {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = f16_bits_to_f32(w[i / 2] >> (16 * (i & 1)));
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      f[i] = (i & 1) ? __uint_as_float(w[i / 2] & 0xffff0000u) : __uint_as_float(w[i / 2] << 16);
  } else {
    static_assert(DT == DT_FP8, "dtype");
#pragma unroll
    for (int wi = 0; wi < (N + 3) / 4; ++wi) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[wi]), false);
      f[4 * wi] = lo.x;
      if (4 * wi + 1 < N) f[4 * wi + 1] = lo.y;
      if (4 * wi + 2 < N) {
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[wi]), true);
        f[4 * wi + 2] = hi.x;
        if (4 * wi + 3 < N) f[4 * wi + 3] = hi.y;
      }
    }
  }
}

// ---- fp32 -> OCP E4M3 code (the fp8 cache write) ------------------------------------------
// |y| -> OCP E4M3 magnitude code, with the sign bit taken from x (the value before division by
// the positive block scale, so a NaN quotient cannot lose its sign): round to nearest, ties to the
// even mantissa; |y| >= 448 (and infinity) saturates to 448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y, float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const uint32_t a = __float_as_uint(y) & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  const float fa = __uint_as_float(a);
  if (fa >= 448.0f) return sign | 0x7eu;
  if (fa < 0.015625f) {
    // below the smallest normal 2^-6 the codes step by 2^-9: scale by 2^9 (exact) and round half
    // to even; a result of 8 is the smallest normal's code 0x08.
    return sign | static_cast<uint32_t>(__builtin_rintf(fa * 512.0f));
  }
  // keep 3 mantissa bits of the fp32 pattern, rounding half to even at bit 20; a carry moves
  // into the exponent, which is then rebiased from 127 to 7.
  const uint32_t rnd = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((((rnd >> 23) - 120u) << 3) | ((rnd >> 20) & 7u));
}

// ---- fp32 -> 16-bit storage ---------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16_rne(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Stores one fp32 result as out_dtype (F32, F16 or BF16).
__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int out_dtype) {
  if (out_dtype == DT_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if (out_dtype == DT_F16) {
    reinterpret_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_f16_rne(v));
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_rne(v));
  }
}

// Stores 4 consecutive fp32 results (idx a multiple of 4) as out_dtype in one vector store.
__device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 v, int out_dtype) {
  if (out_dtype == DT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = v;
  } else {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = out_dtype == DT_F16 ? f32_to_f16_rne(v[i]) : f32_to_bf16_rne(v[i]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) =
        u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

// Work-group barrier for hand-offs through LDS only: orders LDS accesses (this wave's complete
// before the barrier) but does not wait for the wave's outstanding global stores, which nothing
// in the work-group reads back (a store of a new token's rows into the cache, say).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- DPP reductions inside one 16-lane row -------------------------------------------------------
// quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (swaps the two
// quads of each 8-lane half), row_mirror (swaps the two halves): after the four steps every lane
// of the row holds the same row-wide result (each step combines a value with its mirror image,
// and + / max are commutative, so all lanes round identically).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// ---- argument blocks ------------------------------------------------------------------------------
struct DecodeArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  const float* k_scale;
  const float* v_scale;
  // Partial results, one slot per (unit, partition) -- fixed partitions: slot
  // (s * units + x) * max_parts + p; balanced split: slot 2 * work-group + {0: its first unit,
  // 1: its last}. A slot holds the unit's heads_per_unit heads: ws_o[slot][head][D] normalised
  // outputs and ws_ml[slot][head] = (max of log2-scaled scores, sum of exp2).
  float* ws_o;
  float2* ws_ml;
  int* ws_pref;    // balanced split: block prefix sums [S + 1] (written by work-group 0)
  int num_seqs, num_heads, num_kv_heads, max_blocks, num_blocks;
  int part_blocks, max_parts, out_dtype;
  int stream_kv;   // 1: K/V read non-temporally; 0: through the caches (shared blocks)
  int heads_per_unit;  // query heads one work-group accumulates: 1 (VALU) or Hq / Hkv (MFMA)
  int balanced;    // 1: balanced split over nw work-groups; 0: fixed partitions
  int nw;
  int nw_cls;      // balanced split: CUs of a grid of three work-groups per CU (weighted shares), or 0
  int ordered;     // fixed partitions, MFMA kernel: 1-D grid over the ordered work list
  float zscale;    // softmax scale * log2(e)
  // pa_decode_append: the batch's new tokens ([S][Hkv][D], the cache dtype, or the query dtype for
  // an fp8 cache) and their slots; each kernel takes sequence s's new token from here at position
  // L-1. With tail_wgs > 0 (the vector-ALU kernel's ordered 1-D grid) the last tail_wgs
  // work-groups (from index tail_from on; the hardware dispatches them last) write the new tokens
  // into the cache; otherwise the work-group holding the token's block does. nullptr: plain
  // decode.
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  int tail_from, tail_wgs;
  // pa_decode_grouped: sequences group_start[i] .. group_start[i+1]-1 form group i and share
  // their first prefix_blocks[s] table entries. Partial results then sit in one slot per
  // (sequence, query head, part): ws_o[(s * Hq + h) * max_parts + k][D] (heads_per_unit 1), the
  // parts being the prefix partitions followed by the sequence's own; ws_count[s] = their number.
  int grouped;
  int num_groups;
  const int32_t* group_start;
  const int32_t* prefix_blocks;
  int* ws_count;
};

// Chunked prefill: sequence s owns query rows query_start[s] .. query_start[s+1]-1 of q / out
// ([num_tokens][num_heads][D]) and attends lens[s] cached tokens, its new tokens being the last.
struct PrefillArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* query_start;
  const float* k_scale;
  const float* v_scale;
  int num_seqs, num_tokens, num_heads, num_kv_heads, max_blocks, num_blocks, out_dtype;
  int num_tiles;   // row tiles per (sequence, kv head): the longest chunk's rows / rows per tile
  float zscale;    // softmax scale * log2(e)
};

}  // namespace pa
