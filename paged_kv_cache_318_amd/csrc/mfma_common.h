// gfx950 building blocks shared by the matrix-core attention kernels: the 16x16x32 16-bit MFMA,
// exact OCP E4M3 -> 16-bit conversion, fp32 <-> 16-bit rounding, the dim layout of the score
// operands, and the direct global -> LDS load.
#pragma once

#include "pa_device.h"

namespace pa {

template <int QDT>
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QDT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two OCP E4M3 codes (bytes 0-1 of `w`, or 2-3 when HI) -> two packed 16-bit values of the
// MFMA input type, with gfx950's scaled converter at scale 1.0: one instruction, exact (every
// E4M3 value is representable in bf16 and fp16).
template <int QDT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to16(uint32_t w) {
  if constexpr (QDT == DT_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

template <int QDT>
__device__ __forceinline__ uint32_t to16(float x) {
  if constexpr (QDT == DT_BF16) return f32_to_bf16_rne(x);
  else return f32_to_f16_rne(x);
}
template <int QDT>
__device__ __forceinline__ float from16(uint32_t b) {
  if constexpr (QDT == DT_BF16) return bf16_bits_to_f32(b);
  else return f16_bits_to_f32(b);
}

// Two fp32 values -> two packed 16-bit values of the MFMA input type (lo in bits 0-15), rounded
// to nearest even by gfx950's packed converters (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int QDT>
__device__ __forceinline__ uint32_t pack16x2(float a, float b) {
  const f32x2 v{a, b};
  if constexpr (QDT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
template <int QDT>
__device__ __forceinline__ float lo16_to_f32(uint32_t w) { return from16<QDT>(w & 0xffffu); }
template <int QDT>
__device__ __forceinline__ float hi16_to_f32(uint32_t w) { return from16<QDT>(w >> 16); }

// (a, b) -> hi: both rounded to the 16-bit type; lo: the two rounding remainders, rounded too.
// hi + lo carries a and b to about 16 significant bits. For bf16 each remainder is one dot2
// instruction, hi . (-1, 0) + a and hi . (0, -1) + b: both products are exact and the remainder
// of a rounding to bf16 is an fp32 number (bf16 has fp32's exponent range), so the sum is exact.
template <int QDT>
__device__ __forceinline__ void split16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack16x2<QDT>(a, b);
  if constexpr (QDT == DT_BF16) {
    // (-1, 0) goes through a scalar register: as an operand of this instruction the compiler
    // encodes it as the inline constant -1.0, which the hardware does not read as that pair
    uint32_t m1_lo;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(m1_lo));
    const bf16x2_t h = __builtin_bit_cast(bf16x2_t, hi);
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, m1_lo), a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, 0xbf800000u), b, false);
    lo = pack16x2<QDT>(ra, rb);
  } else {
    lo = pack16x2<QDT>(a - lo16_to_f32<QDT>(hi), b - hi16_to_f32<QDT>(hi));
  }
}

// First of the 8 contiguous dims lane group q4 contributes to score MFMA kk: 16-bit keys load
// 16 bytes (8 dims) per MFMA at byte 64*kk + 16*q4 of the row; fp8 keys load 16 bytes (16 dims,
// two MFMAs) at byte 64*(kk/2) + 16*q4.
template <int EB>
__device__ __forceinline__ constexpr int dim_base(int q4, int kk) {
  return EB == 2 ? 32 * kk + 8 * q4 : 64 * (kk / 2) + 16 * q4 + 8 * (kk % 2);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// gfx950 direct global -> LDS load: each lane's 16 bytes at `src` land at lds_base + 16 * lane.
template <int AUX>
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds_base, 16, 0, AUX);
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) of a wave64 in registers, with
// gfx950's permlane swaps: called with the same value as both operands, a swap returns the pair
// {x[l], x[l ^ 16]} (or {x[l], x[l ^ 32]}) in its two results, in some order -- no LDS round
// trip as with a lane shuffle. max and + are commutative, so the order does not matter.
__device__ __forceinline__ float pair16_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

}  // namespace pa
