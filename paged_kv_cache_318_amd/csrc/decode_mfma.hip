// Decode-step paged attention for grouped-query heads on gfx950 matrix cores.
//
// Same result as the VALU variant ("PagedAttention", Wikipedia article, section "Математическая
// формулировка": causal attention of the newest token, taken block by block through the table).
// Grouped-query attention ("PagedAttention", Ultralytics glossary, section "関連手法") lets the
// G query heads of one kv head share every key/value block, so the work for one (kv head,
// block) is a small dense contraction:
//     Z^T[16 tokens][G heads]  = K_tile[16][D] . Q_g^T[D][G]        (scores)
//     O^T[D][G]               += V_tile^T[D][16] . P^T[16][G]        (weighted values)
// One work-group (4 wave64s) handles one (kv head, sequence, partition); wave w takes blocks
// w, w+4, ... of the partition, so each K/V tile is fetched from HBM once for all G heads.
//
// Operand layouts (v_mfma_f32_16x16x32_{bf16,f16} and v_mfma_f32_16x16x16{bf16_1k,f16}):
//   lane = 16*q4 + n. Scores: A = keys, row n = token n, lane group q4 supplies 8 dims per
//   MFMA (dims q4*D/4 + 8*kk .. +8, one contiguous D/4-dim run per lane per tile); B = queries,
//   column n = head n of the group (zero for n >= G), same dims. The 16x16 result gives lane
//   (q4, n) the scores of tokens 4*q4 .. 4*q4+3 for head n -- exactly the B operand a 16x16x16
//   MFMA wants for P^T (k = tokens 4*q4.., column n). Values are stored dim-major in a block, so
//   the A operand of the value product (row = dim 16*mi + n, k = tokens 4*q4 .. 4*q4+3) is one
//   contiguous 8-byte (16-bit cache) or 4-byte (fp8) load. No lane shuffles are needed between
//   the two products; only the running max crosses the four lane groups (two xor shuffles).
// The weights P are fed to the MFMA as a 16-bit hi part plus a 16-bit remainder (two MFMAs), so
// they carry ~16 significant bits instead of 8 (bf16) or 11 (fp16).
// fp8 caches: codes are converted exactly to the MFMA input type; the per-(block, kv head) key
// scale multiplies the scores and the value scale multiplies P, never the codes.

#include "pa_device.h"
#include "pa_launch.h"

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

template <int QDT>
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (QDT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Two fp32 values that are exactly representable in the 16-bit type -> one packed word.
template <int QDT>
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  if constexpr (QDT == DT_BF16)
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  else
    return f32_to_f16_rne(lo) | (f32_to_f16_rne(hi) << 16);
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

template <int CDT, int QDT, int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int B = 16;
  constexpr int EB = Elem<CDT>::bytes;
  constexpr int KK = D / 32;  // score MFMAs per tile
  constexpr int MI = D / 16;  // value MFMA tiles (x2 for hi / remainder)
  constexpr int DQ = D / 4;   // contiguous key dims per lane group
  extern __shared__ float smem[];
  const int g = blockIdx.x, s = blockIdx.y, p = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, n = lane & 15;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  const int nblk = (L + B - 1) / B;
  const int b0 = p * a.part_blocks;
  if (b0 >= nblk) {
    if (p == 0)
      for (int idx = tid; idx < G * D; idx += 256)
        store_out(a.out, (static_cast<size_t>(s) * Hq + g * G) * D + idx, 0.0f, a.out_dtype);
    return;
  }
  const int b1 = min(nblk, b0 + a.part_blocks);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

  u32x4 qop[KK];
  if (n < G) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(a.q) +
        ((static_cast<size_t>(s) * Hq + g * G + n) * D + q4 * DQ) * 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = qp[kk];
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 acc[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), lsum = 0.0f;

  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const size_t tile = static_cast<size_t>(B) * D * EB;
  for (int j = b0 + wave; j < b1; j += 4) {
    int pb = trow[j];
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    const size_t base = (static_cast<size_t>(pb) * Hkv + g) * tile;
    const uint8_t* kt = a.k_cache + base;
    const uint8_t* vt = a.v_cache + base;
    const Raw<DQ * EB> kr = load_raw<DQ * EB>(kt + (n * D + q4 * DQ) * EB);
    Raw<4 * EB> vr[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) vr[mi] = load_raw<4 * EB>(vt + ((16 * mi + n) * B + 4 * q4) * EB);

    float zs = a.zscale, vs = 1.0f;
    if constexpr (CDT == DT_FP8) {
      zs *= a.k_scale[static_cast<size_t>(pb) * Hkv + g];
      vs = a.v_scale[static_cast<size_t>(pb) * Hkv + g];
    }

    // scores
    f32x4 zt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 kop;
      if constexpr (EB == 2) {
        kop = u32x4{kr.w[4 * kk], kr.w[4 * kk + 1], kr.w[4 * kk + 2], kr.w[4 * kk + 3]};
      } else {
        float f[8];
        to_f32<DT_FP8, 8>(&kr.w[2 * kk], f);
        kop = u32x4{pack_exact<QDT>(f[0], f[1]), pack_exact<QDT>(f[2], f[3]),
                    pack_exact<QDT>(f[4], f[5]), pack_exact<QDT>(f[6], f[7])};
      }
      zt = mfma_k32<QDT>(kop, qop[kk], zt);
    }
    const int valid = L - j * B - 4 * q4;  // this lane group's tokens below L
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (i < valid) ? zt[i] * zs : neg_inf();
    float tm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m, tm);  // finite: every block of the sequence holds a valid token
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float pz[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pz[i] = __builtin_amdgcn_exp2f(z[i] - mn);
      psum += pz[i];
    }
    lsum = lsum * alpha + psum;
    m = mn;

    // P^T operand: hi part and remainder
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = pz[i] * vs;
      hb[i] = to16<QDT>(pv);
      lb[i] = to16<QDT>(pv - from16<QDT>(hb[i]));
    }
    const u32x2 phi = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    const u32x2 plo = u32x2{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};

    // weighted values; tokens at or beyond L get zero values (their weights are already 0)
    const uint32_t mk0 = valid >= 2 ? 0xffffffffu : (valid == 1 ? 0x0000ffffu : 0u);
    const uint32_t mk1 = valid >= 4 ? 0xffffffffu : (valid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      u32x2 vop;
      if constexpr (EB == 2) {
        vop = u32x2{vr[mi].w[0], vr[mi].w[1]};
      } else {
        float f[4];
        to_f32<DT_FP8, 4>(vr[mi].w, f);
        vop = u32x2{pack_exact<QDT>(f[0], f[1]), pack_exact<QDT>(f[2], f[3])};
      }
      vop.x &= mk0;
      vop.y &= mk1;
      f32x4 t = acc[mi] * alpha;
      t = mfma_k16<QDT>(vop, phi, t);
      acc[mi] = mfma_k16<QDT>(vop, plo, t);
    }
  }

  // per-column sum over the four lane groups, then merge the four waves through LDS
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  float* sm_m = smem;
  float* sm_l = smem + 64;
  float* sm_o = smem + 128;  // [4 waves][G][D]
  if (q4 == 0) {
    sm_m[wave * 16 + n] = m;
    sm_l[wave * 16 + n] = lsum;
  }
  if (n < G) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[(wave * G + n) * D + 16 * mi + 4 * q4 + i] = acc[mi][i];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int nn = idx / D, d = idx - (idx / D) * D;
    float M = sm_m[nn];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + nn]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w * 16 + nn];
      const float e = (mw == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      num = __builtin_fmaf(e, sm_o[(w * G + nn) * D + d], num);
      den = __builtin_fmaf(e, sm_l[w * 16 + nn], den);
    }
    const int h = g * G + nn;
    const float o = num / den;
    if (nparts == 1) {
      store_out(a.out, (static_cast<size_t>(s) * Hq + h) * D + d, o, a.out_dtype);
    } else {
      const size_t pi = (static_cast<size_t>(s) * Hq + h) * a.max_parts + p;
      a.ws_o[pi * D + d] = o;
      if (d == 0) a.ws_ml[pi] = make_float2(M, den);
    }
  }
}

template <int CDT, int QDT>
static hipError_t launch_mfma_d(const DecodeArgs& a, int D, hipStream_t st) {
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
  const int G = a.num_heads / a.num_kv_heads;
  const size_t shm = (128 + static_cast<size_t>(4) * G * D) * sizeof(float);
  if (D == 64) hipLaunchKernelGGL((decode_mfma_kernel<CDT, QDT, 64>), grid, dim3(256), shm, st, a);
  else if (D == 128) hipLaunchKernelGGL((decode_mfma_kernel<CDT, QDT, 128>), grid, dim3(256), shm, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int cdt, int qdt, int D, hipStream_t st) {
  if (cdt == DT_F16 && qdt == DT_F16) return launch_mfma_d<DT_F16, DT_F16>(a, D, st);
  if (cdt == DT_BF16 && qdt == DT_BF16) return launch_mfma_d<DT_BF16, DT_BF16>(a, D, st);
  if (cdt == DT_FP8 && qdt == DT_F16) return launch_mfma_d<DT_FP8, DT_F16>(a, D, st);
  if (cdt == DT_FP8 && qdt == DT_BF16) return launch_mfma_d<DT_FP8, DT_BF16>(a, D, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
