// Decode-step paged attention, VALU variant, and the partition merge kernel (gfx950).
//
// What is computed ("PagedAttention", Wikipedia article, section "Математическая формулировка"):
// for the newest query token of sequence s and query head h, the causal softmax attention over
// the L = context_lens[s] cached tokens, evaluated block by block as in the page's blockwise
// form -- block j of B tokens read from the physical block block_tables[s][j] ("PagedAttention",
// Ultralytics glossary, section "ページングの仕組み": the kernel follows the table block by
// block). The blockwise denominator is one sum over all blocks; here it is accumulated as an
// online (running-max) softmax, and partitions of a long sequence are combined by an exact
// log-sum-exp merge, which regroups that same sum.
//
// Mapping (one work-group = 4 wave64s = one (query head, sequence, partition)):
//   * wave w takes the partition's blocks w, w+4, w+8, ... (logical order fixed, so the result
//     does not depend on where the blocks sit in the pool);
//   * inside a wave, 16-lane row r owns tokens r*B/4 .. r*B/4 + B/4-1 of every block; lane c of
//     the row owns key dims c*D/16 .. c*D/16 + D/16-1 (one 16-byte load per token for a 16-bit
//     D=128 cache, so the four rows read 4 x 256 B per instruction) and value dims c, c+16, ...
//     (values are dim-major in the block, so a lane reads the row's B/4 tokens of one dim);
//   * q.k partial sums are reduced across the row with four DPP steps; each row keeps its own
//     running max / sum / accumulator, merged with the other rows and waves through LDS at the
//     end (the same merge algebra as across partitions).
// Scores are kept in the log2 domain: z = (q.k) * scale * log2(e), weights exp2(z - max).
// Tokens at or beyond L in the last block are excluded by selects (never by multiplying by 0),
// so whatever sits in unused slots -- NaN included -- cannot reach the output.

#include "kv_write.h"
#include "pa_device.h"
#include "pa_launch.h"
#include "pa_sched.h"

namespace pa {

// Blocks whose loads a wave issues together before their math (tiles in flight per wave).
constexpr int kValuBlocksPerIter = 2;

// NT: read K/V tiles non-temporally (streaming; the default) or through the caches (when blocks
// are shared between sequences of the batch and a tile fetched for one is reused by another).
// Grid (query head, sequence, partition), or with a.ordered a 1-D grid over the ordered work list
// (longest work first), its (item, query head) pairs, query head fastest, handed out with the
// odd-numbered XCDs taking 8 for every 9 the even ones take (pa_sched.h); the lengths staged in
// dynamic LDS.
template <int CDT, int QDT, int D, int B, bool NT>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int EB = Elem<CDT>::bytes;
  constexpr int QB = Elem<QDT>::bytes;
  constexpr int DPL = D / 16;  // key dims per lane
  constexpr int TPR = B / 4;   // tokens per 16-lane row
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r = lane >> 4, c = lane & 15;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  if (a.tail_wgs > 0 && static_cast<int>(blockIdx.x) >= a.tail_from) {  // pa_decode_append's writes
    tail_write<CDT, CDT == DT_FP8 ? QDT : CDT, D, B>(a, static_cast<int>(blockIdx.x) - a.tail_from);
    return;
  }

  int h, s, p, L;
  if (a.ordered) {
    extern __shared__ int order_lds[];
    const long long unit = xcd_weighted_item(blockIdx.x);
    if (unit < 0) return;  // an odd-numbered XCD's empty work-group
    h = static_cast<int>(unit % Hq);
    const int2 it = ordered_item(a, B, unit / Hq, order_lds);
    if (it.x < 0) return;
    s = __builtin_amdgcn_readfirstlane(it.x);
    p = __builtin_amdgcn_readfirstlane(it.y);
    L = __builtin_amdgcn_readfirstlane(order_lds[s]);
  } else {
    h = blockIdx.x;
    s = blockIdx.y;
    p = blockIdx.z;
    L = a.lens[s];
    L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  }
  const int nblk = (L + B - 1) / B;
  const int b0 = p * a.part_blocks;
  const size_t orow = (static_cast<size_t>(s) * Hq + h) * D;
  if (b0 >= nblk) {
    if (p == 0 && tid < D) store_out(a.out, orow + tid, 0.0f, a.out_dtype);  // L == 0
    return;
  }
  const int b1 = min(nblk, b0 + a.part_blocks);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  const int g = h / (Hq / Hkv);
  // pa_decode_append: the partition holding the last block substitutes the new token (position
  // L-1, offset o_new of that block) for what the cache holds there, in the registers its tile
  // was loaded into. Without tail writers (3-D grid) it also -- one work-group per kv head --
  // stores the key row and the whole value tile back (whole lines rather than one element per
  // dim row).
  constexpr int NDT = CDT == DT_FP8 ? QDT : CDT;  // dtype of the new rows
  constexpr int NEB = Elem<NDT>::bytes;
  const int slot_new = (a.new_slots != nullptr && b1 == nblk) ? new_token_slot(a, s, L, B) : -1;
  const int o_new = (L - 1) % B;
  const bool writer = h % (Hq / Hkv) == 0;

  // query dims c*DPL .. c*DPL+DPL-1, as fp32
  float qf[DPL];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + (orow + c * DPL) * QB;
    Raw<DPL * QB> qr = load_raw<DPL * QB>(qp);
    to_f32<QDT, DPL>(qr.w, qf);
  }

  float m = neg_inf(), l = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;

  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const size_t tile = static_cast<size_t>(B) * D * EB;  // bytes of one (block, head) tile
  // this wave's blocks are b0 + wave + 4*i; their table entries are fetched 64 at a time into
  // one VGPR (lane i holds entry i) and read back with readlane, off the per-tile latency chain
  const int nmine = b0 + wave < b1 ? (b1 - b0 - wave + 3) / 4 : 0;
  for (int base_i = 0; base_i < nmine; base_i += 64) {
  const int cnt = min(64, nmine - base_i);
  int tv = 0;
  if (lane < cnt) {
    tv = trow[b0 + wave + 4 * (base_i + lane)];
    tv = tv < 0 ? 0 : (tv >= a.num_blocks ? a.num_blocks - 1 : tv);
  }
  for (int it = 0; it < cnt; it += kValuBlocksPerIter) {
    // issue the loads of up to kValuBlocksPerIter blocks before any of their math, so each wave
    // keeps that many tiles in flight
    Raw<DPL * EB> kr[kValuBlocksPerIter][TPR];
    Raw<TPR * EB> vr[kValuBlocksPerIter][DPL];
    int pbs[kValuBlocksPerIter];
    Raw<DPL * NEB> knew;
    uint32_t vnew[DPL];
#pragma unroll
    for (int u = 0; u < kValuBlocksPerIter; ++u) {
      if (it + u >= cnt) break;
      pbs[u] = __builtin_amdgcn_readlane(tv, it + u);
      const size_t base = (static_cast<size_t>(pbs[u]) * Hkv + g) * tile;
      const uint8_t* kt = a.k_cache + base;
      const uint8_t* vt = a.v_cache + base;
      // each key load covers whole token rows (16 lanes x D/16 dims) and each value load whole
      // dim rows of the block, so full cache lines
#pragma unroll
      for (int i = 0; i < TPR; ++i)
        kr[u][i] = load_raw<DPL * EB, NT>(kt + ((r * TPR + i) * D + c * DPL) * EB);
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj)
        vr[u][jj] = load_raw<TPR * EB, NT>(vt + ((c + 16 * jj) * B + r * TPR) * EB);
      if (slot_new >= 0 && b0 + wave + 4 * (base_i + it + u) == nblk - 1) {
        // the new token's rows, fetched along with the tile they go into
        const size_t row = (static_cast<size_t>(s) * Hkv + g) * D;
        knew = load_raw<DPL * NEB>(reinterpret_cast<const uint8_t*>(a.k_new) + (row + c * DPL) * NEB);
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) {
          if constexpr (NEB == 4) vnew[jj] = reinterpret_cast<const uint32_t*>(a.v_new)[row + c + 16 * jj];
          else vnew[jj] = reinterpret_cast<const uint16_t*>(a.v_new)[row + c + 16 * jj];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kValuBlocksPerIter; ++u) {
    if (it + u >= cnt) break;
    const int j = b0 + wave + 4 * (base_i + it + u);
    const int pb = pbs[u];
    float zs = a.zscale;
    float vs = 1.0f;
    if constexpr (CDT == DT_FP8) {
      zs *= a.k_scale[static_cast<size_t>(pb) * Hkv + g];
      vs = a.v_scale[static_cast<size_t>(pb) * Hkv + g];
    }
    const int valid = L - j * B - r * TPR;  // tokens of this row below L (may be <= 0 or > TPR)
    if (slot_new >= 0 && j == nblk - 1) {
      float ks = 1.0f, vsc = 1.0f;
      if constexpr (CDT == DT_FP8) {
        ks = a.k_scale[static_cast<size_t>(pb) * Hkv + g];
        vsc = vs;
      }
      const Raw<DPL * EB> kc = new_key_piece<CDT, NDT, DPL>(knew, ks);
      const int rn = o_new / TPR, en = o_new - rn * TPR;  // row and element holding the token
#pragma unroll
      for (int i = 0; i < TPR; ++i)
        if (r == rn && i == en) kr[u][i] = kc;
      if (r == rn) {
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) put_elem<EB>(vr[u][jj], en, new_value_bits<CDT, NDT>(vnew[jj], vsc));
      }
      if (writer && a.tail_wgs == 0) {
        const size_t base = (static_cast<size_t>(pb) * Hkv + g) * tile;
        uint8_t* kt = const_cast<uint8_t*>(a.k_cache) + base;
        uint8_t* vt = const_cast<uint8_t*>(a.v_cache) + base;
        if (r == rn) store_raw<DPL * EB>(kt + (o_new * D + c * DPL) * EB, kc);
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) store_raw<TPR * EB>(vt + ((c + 16 * jj) * B + r * TPR) * EB, vr[u][jj]);
      }
    }

    float z[TPR];
#pragma unroll
    for (int i = 0; i < TPR; ++i) {
      float kf[DPL];
      to_f32<CDT, DPL>(kr[u][i].w, kf);
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) dot = __builtin_fmaf(qf[e], kf[e], dot);
      dot = row_sum16(dot);
      z[i] = (i < valid) ? dot * zs : neg_inf();
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < TPR; ++i) mt = fmaxf(mt, z[i]);
    const float mn = fmaxf(m, mt);
    if (mn != neg_inf()) {  // a row that has seen no valid token yet keeps its empty state
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      float pz[TPR];
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < TPR; ++i) {
        pz[i] = __builtin_amdgcn_exp2f(z[i] - mn);
        psum += pz[i];
      }
      l = l * alpha + psum;
      m = mn;
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) {
        float vf[TPR];
        to_f32<CDT, TPR>(vr[u][jj].w, vf);
        float t = acc[jj] * alpha;
        float pv = 0.0f;
#pragma unroll
        for (int i = 0; i < TPR; ++i) pv = __builtin_fmaf(pz[i], (i < valid) ? vf[i] : 0.0f, pv);
        acc[jj] = __builtin_fmaf(pv, vs, t);
      }
    }
    }
  }
  }

  // merge the 16 row states (4 waves x 4 rows) of this work-group
  __shared__ float sm_m[16], sm_l[16];
  __shared__ float sm_acc[16][D + 1];
  const int k = wave * 4 + r;
  if (c == 0) {
    sm_m[k] = m;
    sm_l[k] = l;
  }
#pragma unroll
  for (int jj = 0; jj < DPL; ++jj) sm_acc[k][c + 16 * jj] = acc[jj];
  lds_barrier();
  if (tid < D) {
    float M = sm_m[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) M = fmaxf(M, sm_m[i]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float w = (sm_m[i] == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(sm_m[i] - M);
      num = __builtin_fmaf(w, sm_acc[i][tid], num);
      den = __builtin_fmaf(w, sm_l[i], den);
    }
    const float o = num / den;
    if (nparts == 1) {
      store_out(a.out, orow + tid, o, a.out_dtype);
    } else {
      const size_t pi = (static_cast<size_t>(s) * Hq + h) * a.max_parts + p;
      a.ws_o[pi * D + tid] = o;
      if (tid == 0) a.ws_ml[pi] = make_float2(M, den);
    }
  }
}

// One work-group of D threads per (query head, sequence): combines the partial results of the
// head's unit. With per-part maxima m_k, sums l_k and normalised outputs o_k (log2 domain):
//   out = sum_k w_k o_k / sum_k w_k,   w_k = l_k * exp2(m_k - max_k m_k).
// Fixed partitions: the parts are the unit's partitions in order. Balanced split: the parts are
// the partial results of the work-groups whose shares cut the unit, in share order (a unit held
// whole by one work-group was written by it directly; an empty sequence gets a zero output here).
// The weights are computed once per part into LDS; every thread then sums over parts in the same
// order (deterministic), with the partial-output loads unrolled.
constexpr int kMergeChunk = 1024;
constexpr int kMergeFast = 16;  // units of at most this many parts take the register path

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a, int block_size) {
  __shared__ float sw[kMergeChunk];
  __shared__ float sred[D / 64];
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int gu = a.heads_per_unit, x = h / gu, hn = h - x * gu;
  const long long hu = a.num_heads / gu;
  const size_t orow = (static_cast<size_t>(s) * a.num_heads + h) * D;
  int count;                 // parts to combine
  size_t first_slot = 0;     // fixed partitions: slots first_slot + k
  int i0 = 0;                // balanced split: work-groups i0 .. i0 + count - 1
  bool i0_first = false;     // ... and whether the unit is work-group i0's first unit
  if (a.grouped) {  // pa_decode_grouped: every part is a partial result, prefix parts first
    count = a.ws_count[s];
    if (count <= 0) {
      store_out(a.out, orow + d, 0.0f, a.out_dtype);
      return;
    }
    first_slot = (static_cast<size_t>(s) * a.num_heads + h) * a.max_parts;
  } else if (a.balanced) {
    const int p0 = a.ws_pref[s], nb = a.ws_pref[s + 1] - p0;
    if (nb == 0) {
      store_out(a.out, orow + d, 0.0f, a.out_dtype);
      return;
    }
    const long long W = static_cast<long long>(a.ws_pref[a.num_seqs]) * hu;
    const int nw = balanced_groups(W, a.nw);
    const long long ustart = static_cast<long long>(p0) * hu + static_cast<long long>(x) * nb;
    i0 = share_owner(W, nw, a.nw_cls, ustart);
    const int i1 = share_owner(W, nw, a.nw_cls, ustart + nb - 1);
    if (i0 == i1) return;  // one work-group took the whole unit and wrote its output
    count = i1 - i0 + 1;   // every share is non-empty, so each of these holds a partial result
    i0_first = share_lo(W, nw, a.nw_cls, i0) == ustart;
  } else {
    int L = a.lens[s];
    L = L < 0 ? 0 : (L > a.max_blocks * block_size ? a.max_blocks * block_size : L);
    const int nblk = (L + block_size - 1) / block_size;
    count = (nblk + a.part_blocks - 1) / a.part_blocks;
    if (count <= 1) return;
    first_slot = (static_cast<size_t>(s) * hu + x) * a.max_parts;
  }
  auto slot_of = [&](int k) -> size_t {
    if (a.grouped || !a.balanced) return first_slot + k;
    return k == 0 ? static_cast<size_t>(2 * i0 + (i0_first ? 0 : 1)) : static_cast<size_t>(2 * (i0 + k));
  };
  if (count <= kMergeFast) {
    // few parts (the usual case): every (max, sum) and output load of the unit is issued at once,
    // then the same sums as below in the same order (bit-identical to the general path)
    float2 ml[kMergeFast];
    float o[kMergeFast];
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) {
      if (k < count) {
        const size_t sl = slot_of(k) * gu + hn;
        ml[k] = a.ws_ml[sl];
        o[k] = a.ws_o[sl * D + d];
      }
    }
    float M = neg_inf();
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k)
      if (k < count) M = fmaxf(M, ml[k].x);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) {
      if (k < count) {
        const float wk = ml[k].y * __builtin_amdgcn_exp2f(ml[k].x - M);
        den += wk;
        num = __builtin_fmaf(wk, o[k], num);
      }
    }
    store_out(a.out, orow + d, num / den, a.out_dtype);
    return;
  }
  float M = neg_inf();
  for (int k = d; k < count; k += D) M = fmaxf(M, a.ws_ml[slot_of(k) * gu + hn].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((d & 63) == 0) sred[d >> 6] = M;
  __syncthreads();
  M = sred[0];
#pragma unroll
  for (int i = 1; i < D / 64; ++i) M = fmaxf(M, sred[i]);
  float num = 0.0f, den = 0.0f;
  for (int c0 = 0; c0 < count; c0 += kMergeChunk) {
    const int n = min(kMergeChunk, count - c0);
    for (int k = d; k < n; k += D) {
      const float2 ml = a.ws_ml[slot_of(c0 + k) * gu + hn];
      sw[k] = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < n; ++k) {
      const float wk = sw[k];
      den += wk;
      num = __builtin_fmaf(wk, a.ws_o[(slot_of(c0 + k) * gu + hn) * D + d], num);
    }
    __syncthreads();
  }
  store_out(a.out, orow + d, num / den, a.out_dtype);
}

// ---- launchers ----------------------------------------------------------------------------------
template <int CDT, int QDT, int D, int B>
static void launch_valu_nt(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  const size_t shm = a.ordered ? static_cast<size_t>(ordered_lds_ints(a.num_seqs)) * sizeof(int) : 0;
  if (a.stream_kv) launch_kernel((decode_valu_kernel<CDT, QDT, D, B, true>), grid, dim3(256), shm, st, a);
  else launch_kernel((decode_valu_kernel<CDT, QDT, D, B, false>), grid, dim3(256), shm, st, a);
}

template <int CDT, int QDT, int D>
static hipError_t launch_valu_b(const DecodeArgs& a, int B, dim3 grid, hipStream_t st) {
  switch (B) {
    case 8: launch_valu_nt<CDT, QDT, D, 8>(a, grid, st); break;
    case 16: launch_valu_nt<CDT, QDT, D, 16>(a, grid, st); break;
    case 32: launch_valu_nt<CDT, QDT, D, 32>(a, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int CDT, int QDT>
static hipError_t launch_valu_d(const DecodeArgs& a, int D, int B, dim3 grid, hipStream_t st) {
  if (D == 64) return launch_valu_b<CDT, QDT, 64>(a, B, grid, st);
  if (D == 128) return launch_valu_b<CDT, QDT, 128>(a, B, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_valu(const DecodeArgs& a0, int cdt, int qdt, int D, int B, hipStream_t st) {
  DecodeArgs a = a0;
  a.tail_from = 0;
  a.tail_wgs = 0;
  const dim3 grid = a.ordered ? dim3(add_tail_writers(a, static_cast<unsigned>(xcd_weighted_grid(
                                    static_cast<long long>(a.num_heads) * a.num_seqs * a.max_parts)), D))
                              : dim3(a.num_heads, a.num_seqs, a.max_parts);
  if (cdt == DT_F32 && qdt == DT_F32) return launch_valu_d<DT_F32, DT_F32>(a, D, B, grid, st);
  if (cdt == DT_F16 && qdt == DT_F16) return launch_valu_d<DT_F16, DT_F16>(a, D, B, grid, st);
  if (cdt == DT_BF16 && qdt == DT_BF16) return launch_valu_d<DT_BF16, DT_BF16>(a, D, B, grid, st);
  if (cdt == DT_FP8 && qdt == DT_F16) return launch_valu_d<DT_FP8, DT_F16>(a, D, B, grid, st);
  if (cdt == DT_FP8 && qdt == DT_BF16) return launch_valu_d<DT_FP8, DT_BF16>(a, D, B, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeArgs& a, int D, int B, hipStream_t st) {
  const dim3 grid(a.num_heads, a.num_seqs);
  if (D == 64) launch_kernel((decode_merge_kernel<64>), grid, dim3(64), 0, st, a, B);
  else if (D == 128) launch_kernel((decode_merge_kernel<128>), grid, dim3(128), 0, st, a, B);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
