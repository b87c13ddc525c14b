// Causal paged attention of a chunk of new query tokens per sequence (prefill of the chunk over
// the cached context) on gfx950 matrix cores.
//
// The equations of "PagedAttention" (Wikipedia article, section "Математическая формулировка")
// hold for any query position i: query token i attends the keys at positions 1..i, read block by
// block through the table, the last block cut at i. A chunk of n new tokens of a sequence holding
// L tokens (the chunk's keys and values already written) has queries at positions L-n .. L-1.
//
// Rows: the n * G (query token, query head of the kv group) pairs of one (sequence, kv head),
// token-major. One work-group (4 wave64s) takes 64 consecutive rows, each wave 16 of them as the
// 16 columns of the same 16x16x32 MFMA the decode kernel uses:
//     Z^T[16 tokens][16 rows]  = K_tile[16][D] . Q^T[D][16 rows]        (scores)
//     O^T[D][16 rows]         += V^T[D][32 tokens] . P^T[32 tokens][16 rows]
// so every K/V tile is fetched once per 64 rows. Per iteration the work-group stages two blocks'
// key and value tiles (16 KB at 16 bits) in LDS with gfx950's direct global -> LDS loads (1 KB
// contiguous per load instruction; keys XOR-swizzled by row so the MFMA-layout reads hit distinct
// banks), then every wave runs its scores, its online softmax and its weighted values out of LDS.
// Each column carries its own causal limit (its query position); a wave's rows never leave it,
// so no cross-wave merge is needed and no workspace either.

#include "mfma_common.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kPrefillRows = 64;  // rows per work-group (4 waves x 16 MFMA columns)

template <int CDT, int D>
constexpr size_t prefill_lds_bytes() {
  return size_t{4} * 16 * D * Elem<CDT>::bytes;  // key tiles of two blocks, then value tiles
}

template <int CDT, int QDT, int D>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int B = 16;
  constexpr int EB = Elem<CDT>::bytes;
  constexpr int KK = D / 32;                 // score MFMAs per block
  constexpr int MI = D / 16;                 // value MFMA tiles (x2 for hi / remainder)
  constexpr int KL = EB == 2 ? KK : KK / 2;  // 16-byte key chunks per lane per block
  constexpr int KT = B * D * EB;             // bytes of one key (or value) tile
  constexpr int CPR = D * EB / 16;           // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;              // key rows per 1 KB load
  constexpr int NCH = KT / 1024;             // 1 KB loads per tile
  static_assert(NCH >= 1 && KT % 1024 == 0, "tile must be a whole number of 1 KB loads");
  extern __shared__ float smem[];
  uint8_t* kt = reinterpret_cast<uint8_t*>(smem);  // [2][KT] keys of the iteration's blocks
  uint8_t* vt = kt + 2 * KT;                       // [2][KT] values (dim-major, as stored)

  const int tile = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, n = lane & 15;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  int q0 = a.query_start[s], q1 = a.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.num_tokens ? a.num_tokens : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.num_tokens ? a.num_tokens : q1);
  const int ns = (q1 - q0) < L ? (q1 - q0) : L;  // a chunk cannot be longer than the sequence
  const int rows = ns * G;
  const int r0 = tile * kPrefillRows;
  if (r0 >= rows) return;
  const int rlast = (r0 + kPrefillRows < rows ? r0 + kPrefillRows : rows) - 1;
  const int nblk = (L - ns + rlast / G) / B + 1;   // blocks up to the group's last query

  // this lane's column: row r = (token k of the chunk, head hh of the group); rows past the
  // chunk attend token 0 only (finite, discarded)
  const int r = r0 + wave * 16 + n;
  const bool live = r < rows;
  const int k = live ? r / G : 0;
  const int hh = live ? r - k * G : 0;
  const int pos = live ? L - ns + k : 0;

  u32x4 qop[KK];
  if (live) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(a.q) +
        ((static_cast<size_t>(q0 + k) * Hq + g * G + hh) * D) * 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = qp[dim_base<EB>(q4, kk) / 8];
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = u32x4{0u, 0u, 0u, 0u};
  }

  // Load c (c = wave + 4*i) of the iteration's 4*NCH 1 KB loads: tile c / NCH (0, 1: keys of
  // blocks A, B; 2, 3: their values), part c % NCH of it.
  int ld_tile[NCH], ld_part[NCH], ld_src[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = wave + 4 * i;
    ld_tile[i] = c / NCH;
    ld_part[i] = c - (c / NCH) * NCH;
    if (ld_tile[i] < 2) {  // keys: lane fetches chunk (lane % CPR) ^ (row % CPR) of its row
      const int row = RPI * ld_part[i] + lane / CPR;
      ld_src[i] = row * CPR * 16 + 16 * ((lane % CPR) ^ (row % CPR));
    } else {               // values: plain contiguous 1 KB
      ld_src[i] = ld_part[i] * 1024 + 16 * lane;
    }
  }
  int kread[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) kread[i] = n * CPR * 16 + 16 * ((4 * i + q4) ^ (n % CPR));

  f32x4 acc[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), lsum = 0.0f;

  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  int tv = 0, tbase = -64;
  for (int j0 = 0; j0 < nblk; j0 += 2) {
    if (j0 - tbase >= 64) {  // next 64 table entries into one VGPR, read back with readlane
      tbase = j0;
      tv = 0;
      if (tbase + lane < nblk) {
        tv = trow[tbase + lane];
        tv = tv < 0 ? 0 : (tv >= a.num_blocks ? a.num_blocks - 1 : tv);
      }
    }
    const bool has_b = j0 + 1 < nblk;
    const int pba = __builtin_amdgcn_readlane(tv, j0 - tbase);
    const int pbb = has_b ? __builtin_amdgcn_readlane(tv, j0 + 1 - tbase) : pba;
    const size_t offa = (static_cast<size_t>(pba) * Hkv + g) * KT;
    const size_t offb = (static_cast<size_t>(pbb) * Hkv + g) * KT;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int t = ld_tile[i];
      const uint8_t* src = (t < 2 ? a.k_cache : a.v_cache) + ((t & 1) ? offb : offa) + ld_src[i];
      dma16<0>(src, kt + t * KT + 1024 * ld_part[i]);  // values follow the keys: vt = kt + 2*KT
    }
    float zs[2], vs[2];
    zs[0] = zs[1] = a.zscale;
    vs[0] = vs[1] = 1.0f;
    if constexpr (CDT == DT_FP8) {
      zs[0] *= a.k_scale[static_cast<size_t>(pba) * Hkv + g];
      zs[1] *= a.k_scale[static_cast<size_t>(pbb) * Hkv + g];
      vs[0] = a.v_scale[static_cast<size_t>(pba) * Hkv + g];
      vs[1] = a.v_scale[static_cast<size_t>(pbb) * Hkv + g];
    }
    // this wave's loads have landed (both counters drained), then every wave's have
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x4 zt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      zt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kb = kt + u * KT;
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(kb + kread[i]);
        if constexpr (EB == 2) {
          zt[u] = mfma_k32<QDT>(raw, qop[i], zt[u]);
        } else {
          const u32x4 k0{fp8x2_to16<QDT, false>(raw.x), fp8x2_to16<QDT, true>(raw.x),
                         fp8x2_to16<QDT, false>(raw.y), fp8x2_to16<QDT, true>(raw.y)};
          zt[u] = mfma_k32<QDT>(k0, qop[2 * i], zt[u]);
          const u32x4 k1{fp8x2_to16<QDT, false>(raw.z), fp8x2_to16<QDT, true>(raw.z),
                         fp8x2_to16<QDT, false>(raw.w), fp8x2_to16<QDT, true>(raw.w)};
          zt[u] = mfma_k32<QDT>(k1, qop[2 * i + 1], zt[u]);
        }
      }
    }
    // lane (q4, n) holds tokens t0(u) .. t0(u)+3 of block j0+u for column n
    float z[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t0 = (j0 + u) * B + 4 * q4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        z[4 * u + i] = (t0 + i <= pos && (u == 0 || has_b)) ? zt[u][i] * zs[u] : neg_inf();
    }
    float tm = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tm = fmaxf(tm, z[i]);
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m, tm);  // finite: block 0 holds token 0, which every column attends
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float pz[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pz[i] = __builtin_amdgcn_exp2f(z[i] - mn);
      psum += pz[i];
    }
    lsum = lsum * alpha + psum;
    m = mn;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[mi] = acc[mi] * alpha;

    // weighted values over the 32 tokens of the two blocks; P^T as 16-bit hi part + remainder;
    // slots at or beyond L (never written) get zero values
    uint32_t hbits[8], lbits[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = pz[i] * (i < 4 ? vs[0] : vs[1]);
      hbits[i] = to16<QDT>(pv);
      lbits[i] = to16<QDT>(pv - from16<QDT>(hbits[i]));
    }
    const u32x4 phi{hbits[0] | (hbits[1] << 16), hbits[2] | (hbits[3] << 16),
                    hbits[4] | (hbits[5] << 16), hbits[6] | (hbits[7] << 16)};
    const u32x4 plo{lbits[0] | (lbits[1] << 16), lbits[2] | (lbits[3] << 16),
                    lbits[4] | (lbits[5] << 16), lbits[6] | (lbits[7] << 16)};
    const int va = L - j0 * B - 4 * q4;                   // this lane group's tokens below L
    const int vb = has_b ? L - (j0 + 1) * B - 4 * q4 : 0;
    const uint32_t ma0 = va >= 2 ? 0xffffffffu : (va == 1 ? 0x0000ffffu : 0u);
    const uint32_t ma1 = va >= 4 ? 0xffffffffu : (va == 3 ? 0x0000ffffu : 0u);
    const uint32_t mb0 = vb >= 2 ? 0xffffffffu : (vb == 1 ? 0x0000ffffu : 0u);
    const uint32_t mb1 = vb >= 4 ? 0xffffffffu : (vb == 3 ? 0x0000ffffu : 0u);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int voff = ((16 * mi + n) * B + 4 * q4) * EB;
      uint32_t a0, a1, c0, c1;
      if constexpr (EB == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(vt + voff);
        const u32x2 y = *reinterpret_cast<const u32x2*>(vt + KT + voff);
        a0 = x.x;
        a1 = x.y;
        c0 = y.x;
        c1 = y.y;
      } else {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vt + voff);
        const uint32_t y = *reinterpret_cast<const uint32_t*>(vt + KT + voff);
        a0 = fp8x2_to16<QDT, false>(x);
        a1 = fp8x2_to16<QDT, true>(x);
        c0 = fp8x2_to16<QDT, false>(y);
        c1 = fp8x2_to16<QDT, true>(y);
      }
      const u32x4 vop{a0 & ma0, a1 & ma1, c0 & mb0, c1 & mb1};
      acc[mi] = mfma_k32<QDT>(vop, phi, acc[mi]);
      acc[mi] = mfma_k32<QDT>(vop, plo, acc[mi]);
    }
    __syncthreads();  // every wave is done with the staged tiles before the next loads land
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (live) {
    const size_t orow = (static_cast<size_t>(q0 + k) * Hq + g * G + hh) * D;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out(a.out, orow + 16 * mi + 4 * q4 + i, acc[mi][i] / lsum, a.out_dtype);
  }
}

template <int CDT, int QDT, int D>
static hipError_t launch_prefill_dn(const PrefillArgs& a, int max_query_len, hipStream_t st) {
  const int G = a.num_heads / a.num_kv_heads;
  const long long rows = static_cast<long long>(max_query_len) * G;
  const dim3 grid(static_cast<unsigned>((rows + kPrefillRows - 1) / kPrefillRows), a.num_kv_heads,
                  a.num_seqs);
  const size_t shm = prefill_lds_bytes<CDT, D>();
  hipLaunchKernelGGL((prefill_mfma_kernel<CDT, QDT, D>), grid, dim3(256), shm, st, a);
  return hipGetLastError();
}

template <int CDT, int QDT>
static hipError_t launch_prefill_d(const PrefillArgs& a, int D, int max_query_len, hipStream_t st) {
  if (D == 64) return launch_prefill_dn<CDT, QDT, 64>(a, max_query_len, st);
  if (D == 128) return launch_prefill_dn<CDT, QDT, 128>(a, max_query_len, st);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, int cdt, int qdt, int D, int max_query_len,
                          hipStream_t st) {
  if (cdt == DT_F16 && qdt == DT_F16) return launch_prefill_d<DT_F16, DT_F16>(a, D, max_query_len, st);
  if (cdt == DT_BF16 && qdt == DT_BF16) return launch_prefill_d<DT_BF16, DT_BF16>(a, D, max_query_len, st);
  if (cdt == DT_FP8 && qdt == DT_F16) return launch_prefill_d<DT_FP8, DT_F16>(a, D, max_query_len, st);
  if (cdt == DT_FP8 && qdt == DT_BF16) return launch_prefill_d<DT_FP8, DT_BF16>(a, D, max_query_len, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
