// The slot write of one new token's key and value row piece (shared by the write kernel and the
// decode kernels that take the new token along). Layouts: k_cache [NB][Hkv][B][D] (a token's key
// is a contiguous row), v_cache [NB][Hkv][D][B] (values dim-major in the block), fp8 scales
// [NB][Hkv].
#pragma once

#include "pa_device.h"

namespace pa {

template <int DT> struct Store;
template <> struct Store<DT_F32> { using T = uint32_t; };
template <> struct Store<DT_F16> { using T = uint16_t; };
template <> struct Store<DT_BF16> { using T = uint16_t; };
template <> struct Store<DT_FP8> { using T = uint8_t; };

// One (new token, kv head, 8 consecutive dims) piece: a 16-byte (32-byte for fp32) load of the
// new key and value, one vector store of the key row piece, and (VALUES) 8 element stores down the
// dim-major value column.
template <int IN_DT, int C_DT, bool VALUES>
__device__ __forceinline__ void write_piece(const void* __restrict__ k_new,
                                            const void* __restrict__ v_new,
                                            void* __restrict__ k_cache, void* __restrict__ v_cache,
                                            int t, int slot, int hh, int d0, int Hkv, int D, int B,
                                            const float* __restrict__ k_scale,
                                            const float* __restrict__ v_scale) {
  constexpr int IEB = Elem<IN_DT>::bytes;
  constexpr int CEB = Elem<C_DT>::bytes;
  using CT = typename Store<C_DT>::T;
  const int b = slot / B, o = slot - (slot / B) * B;
  const size_t src = (static_cast<size_t>(t) * Hkv + hh) * D + d0;
  const Raw<8 * IEB> kr = load_raw<8 * IEB>(reinterpret_cast<const uint8_t*>(k_new) + src * IEB);
  const size_t kdst = ((static_cast<size_t>(b) * Hkv + hh) * B + o) * D + d0;  // elements
  const size_t vdst = ((static_cast<size_t>(b) * Hkv + hh) * D + d0) * B + o;
  uint8_t* kc = reinterpret_cast<uint8_t*>(k_cache);
  CT* vc = reinterpret_cast<CT*>(v_cache);
  if constexpr (C_DT == DT_FP8) {
    const float ks = k_scale[static_cast<size_t>(b) * Hkv + hh];
    float kf[8];
    to_f32<IN_DT, 8>(kr.w, kf);
    uint32_t kw[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) kw[e / 4] |= f32_to_e4m3(kf[e] / ks, kf[e]) << (8 * (e & 3));
    *reinterpret_cast<u32x2*>(kc + kdst) = u32x2{kw[0], kw[1]};
    if constexpr (VALUES) {
      const Raw<8 * IEB> vr = load_raw<8 * IEB>(reinterpret_cast<const uint8_t*>(v_new) + src * IEB);
      const float vs = v_scale[static_cast<size_t>(b) * Hkv + hh];
      float vf[8];
      to_f32<IN_DT, 8>(vr.w, vf);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vc[vdst + static_cast<size_t>(e) * B] = static_cast<CT>(f32_to_e4m3(vf[e] / vs, vf[e]));
    }
  } else {
    static_assert(IN_DT == C_DT, "a 16/32-bit cache stores the input bits");
#pragma unroll
    for (int i = 0; i < 8 * CEB / 16; ++i)
      reinterpret_cast<u32x4*>(kc + kdst * CEB)[i] =
          u32x4{kr.w[4 * i], kr.w[4 * i + 1], kr.w[4 * i + 2], kr.w[4 * i + 3]};
    if constexpr (VALUES) {
      const Raw<8 * IEB> vr = load_raw<8 * IEB>(reinterpret_cast<const uint8_t*>(v_new) + src * IEB);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        CT v;
        if constexpr (CEB == 4) v = vr.w[e];
        else v = static_cast<CT>(vr.w[e / 2] >> (16 * (e & 1)));
        vc[vdst + static_cast<size_t>(e) * B] = v;
      }
    }
  }
}

// ---- the new token taken along by a decode kernel (pa_decode_append) ---------------------------

// Slot of sequence s's new token if it is the slot of position L-1 of its table (the only
// position the decode kernels take from k_new / v_new instead of the cache), else -1.
__device__ __forceinline__ int new_token_slot(const DecodeArgs& a, int s, int L, int B) {
  if (a.new_slots == nullptr || L <= 0) return -1;
  const int slot = a.new_slots[s];
  const int pb = a.tables[static_cast<size_t>(s) * a.max_blocks + (L - 1) / B];
  return (slot >= 0 && pb >= 0 && pb < a.num_blocks && slot == pb * B + (L - 1) % B) ? slot : -1;
}

// The slot writes of pa_decode_append done by the grid's tail: thread x of the a.tail_wgs
// work-groups (w = its work-group's place among them) takes the (sequence, kv head, 8-dim piece)
// items x, x + 256 * tail_wgs, ... and writes each piece whose sequence's new token the attention
// takes along (new_token_slot), with pa_write_kv's own piece write, so the cache ends as
// pa_write_kv leaves it. Nothing else of the launch reads those slots: the work-group that loads
// a new token's block puts the token in from k_new / v_new instead.
template <int CDT, int NDT, int D, int B>
__device__ void tail_write(const DecodeArgs& a, int w) {
  constexpr int kPieces = D / 8;
  const long long total = static_cast<long long>(a.num_seqs) * a.num_kv_heads * kPieces;
  const long long stride = static_cast<long long>(a.tail_wgs) * blockDim.x;
  for (long long x = static_cast<long long>(w) * blockDim.x + threadIdx.x; x < total; x += stride) {
    const int d0 = static_cast<int>(x % kPieces) * 8;
    const long long sh = x / kPieces;
    const int hh = static_cast<int>(sh % a.num_kv_heads), s = static_cast<int>(sh / a.num_kv_heads);
    int L = a.lens[s];
    L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
    const int slot = new_token_slot(a, s, L, B);
    if (slot < 0) continue;
    write_piece<NDT, CDT, true>(a.k_new, a.v_new, const_cast<uint8_t*>(a.k_cache),
                                const_cast<uint8_t*>(a.v_cache), s, slot, hh, d0, a.num_kv_heads,
                                D, B, a.k_scale, a.v_scale);
  }
}

// A new token's key piece of N elements (raw input of type NDT) in the cache's representation:
// the input bits for a 16/32-bit cache; for an fp8 cache the E4M3 codes of x / scale, as the
// write kernel stores them.
template <int CDT, int NDT, int N>
__device__ __forceinline__ Raw<N * Elem<CDT>::bytes> new_key_piece(const Raw<N * Elem<NDT>::bytes>& in,
                                                                   float scale) {
  Raw<N * Elem<CDT>::bytes> outp;
  if constexpr (CDT == DT_FP8) {
    float x[N];
    to_f32<NDT, N>(in.w, x);
#pragma unroll
    for (int i = 0; i < (N + 3) / 4; ++i) outp.w[i] = 0u;
#pragma unroll
    for (int e = 0; e < N; ++e) outp.w[e / 4] |= f32_to_e4m3(x[e] / scale, x[e]) << (8 * (e & 3));
  } else {
#pragma unroll
    for (int i = 0; i < (N * Elem<CDT>::bytes + 3) / 4; ++i) outp.w[i] = in.w[i];
  }
  return outp;
}

// One new value element (raw input bits of type NDT) in the cache's representation.
template <int CDT, int NDT>
__device__ __forceinline__ uint32_t new_value_bits(uint32_t in, float scale) {
  if constexpr (CDT == DT_FP8) {
    float x;
    if constexpr (NDT == DT_F32) x = __uint_as_float(in);
    else if constexpr (NDT == DT_F16) x = f16_bits_to_f32(in);
    else x = bf16_bits_to_f32(in);
    return f32_to_e4m3(x / scale, x);
  } else {
    return in;
  }
}

// Element e (a run-time index) of a raw piece of EB-byte elements replaced by `bits`; every word
// is visited with a select, so the piece stays in registers.
template <int EB, int NB>
__device__ __forceinline__ void put_elem(Raw<NB>& r, int e, uint32_t bits) {
  constexpr int PERW = EB >= 4 ? 1 : 4 / EB;  // elements per 32-bit word
  constexpr int NW = NB >= 4 ? NB / 4 : 1;
  const int wi = e / PERW;
  const int sh = (e - wi * PERW) * 8 * EB;
  const uint32_t mask = EB >= 4 ? 0xffffffffu : (((1u << (8 * EB)) - 1u) << sh);
#pragma unroll
  for (int k = 0; k < NW; ++k)
    r.w[k] = (k == wi) ? ((r.w[k] & ~mask) | ((bits << sh) & mask)) : r.w[k];
}

}  // namespace pa
