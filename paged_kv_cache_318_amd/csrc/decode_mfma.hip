// Decode-step paged attention for grouped-query heads on gfx950 matrix cores.
//
// Same result as the VALU variant ("PagedAttention", Wikipedia article, section "Математическая
// формулировка": causal attention of the newest token, taken block by block through the table).
// Grouped-query attention ("PagedAttention", Ultralytics glossary, section "関連手法") lets the
// G query heads of one kv head share every key/value block, so the work for one (kv head,
// block) is a small dense contraction:
//     Z^T[16 tokens][G heads]  = K_tile[16][D] . Q_g^T[D][G]        (scores)
//     O^T[D][G]               += V_tile^T[D][16] . P^T[16][G]        (weighted values)
// One work-group (4 wave64s) handles one (kv head, sequence, partition); wave w takes work items
// (blocks; pairs of blocks at B = 8) w, w+4, ... of the partition, two 16-token tiles per
// iteration, so each K/V tile is fetched from HBM once for all G heads and every wave keeps two
// tiles (16 KB at 16 bits) in flight (fp8 with 16-token blocks: the next iteration's tiles fly
// while this one computes; see mfma_stages_values).
//
// Operand layouts (v_mfma_f32_16x16x32_{bf16,f16}: lane l = 16*q4 + n holds 8 elements of row
// n of A and of column n of B, the k-range given by q4; the 16x16 result gives lane (q4, n) rows
// 4*q4 .. 4*q4+3 of column n):
//   * scores: A = keys (row n = token n of a 16-token tile), B = queries (column n = head n of
//     the group, zero for n >= G); lane group q4 supplies dims dim_base(q4, kk) .. +8 of both, so
//     the contraction pairs the same dims. The result hands lane (q4, n) the scores of tokens
//     4*q4 .. 4*q4+3 of the tile for head n. A tile is a block (B = 16), half of one (B = 32)
//     or a pair of blocks (B = 8).
//   * weighted values over the iteration's two tiles (32 tokens): A = V^T (row = dim
//     16*mi + n), B = P^T (column = head n); lane group q4 supplies tokens 4*q4 .. 4*q4+3 of
//     tile A then of tile B -- exactly the scores it already holds, so no lane shuffles sit
//     between the two products (only the running max crosses the four lane groups). Values are
//     stored dim-major in a block, so each lane's piece is one contiguous 8-byte (16-bit) or
//     4-byte (fp8) load, and one load instruction covers 16 whole dim rows of the tile.
//   * keys are staged through LDS with gfx950's direct global -> LDS loads: every load
//     instruction reads 1 KB of the tile contiguously (whole cache lines, non-temporal) and the
//     MFMA-layout reads come back out of an XOR-swizzled LDS copy. fp8 caches with 16-token
//     blocks stage the value tiles the same way (as stored) and issue each iteration's loads
//     while the iteration before it computes.
// The weights P are fed to the MFMA as a 16-bit hi part plus a 16-bit remainder (two MFMAs), so
// they carry ~16 significant bits instead of 8 (bf16) or 11 (fp16).
// fp8 caches: codes are converted exactly to the MFMA input type; the per-(block, kv head) key
// scale multiplies the scores and the value scale multiplies P, never the codes.

#include "kv_write.h"
#include "mfma_common.h"
#include "pa_device.h"
#include "pa_launch.h"
#include "pa_sched.h"

namespace pa {

// Blocks a wave takes per iteration: two (16 KB of K/V in flight per wave at 16 bits, 8 KB for
// fp8; four fp8 blocks per iteration measured slower).
constexpr int kFp8BlocksPerIter = 2;
constexpr int mfma_blocks_per_iter(int elem_bytes) { return elem_bytes == 2 ? 2 : kFp8BlocksPerIter; }

// fp8 caches with 16-token blocks stage the value tiles through LDS too (next to the keys), so
// that every K/V load of the segment loop is a direct-to-LDS load and the loop can issue each
// iteration's loads one step ahead (fp8 batch: 134.7-135.1 -> 129.7-130.1 us), the keys into a
// ring of two slots (a further 1 us). With register loads in flight beside direct-to-LDS loads
// the compiler drains every load before the first read of a staged tile, which is why the values
// go through LDS too. Per wave: two key slots and one value stage of two tiles, 12 KB (three
// work-groups per CU still fit); at 16 bits the same stages would leave two work-groups per CU.
constexpr bool mfma_stages_values(int cdt, int block_size) { return cdt == DT_FP8 && block_size == 16; }

// Bytes of dynamic LDS: the staged key (and staged value) tiles of one iteration per wave (reused
// by the merge of the four waves at the end of a segment) plus, for the balanced split and the
// ordered fixed partitions, the batch's lengths and prefix sums.
template <int CDT, int D, int B>
constexpr size_t mfma_lds_bytes(int G, int S, bool sched_lds) {
  const size_t stage = size_t{4} * mfma_blocks_per_iter(Elem<CDT>::bytes) * 16 * D * Elem<CDT>::bytes *
                       (mfma_stages_values(CDT, B) ? 3 : 1);
  const size_t merge = (128 + size_t{4} * G * D) * sizeof(float);
  const size_t sched = sched_lds ? static_cast<size_t>(ordered_lds_ints(S)) * sizeof(int) : 0;
  return (stage > merge ? stage : merge) + sched;
}

// One segment: blocks [b0, b1) of unit (sequence s, kv head g) -- all G query heads of the group.
// The result is either the unit's final output (the segment covers all of it) or a partial result
// in workspace slot `slot`. Every thread of the work-group calls it (it synchronises).
// seq0 >= 0 (pa_decode_grouped): the blocks are shared by sequences seq0, seq0 + 1, ..., read
// through sequence s's table, and the rows (MFMA columns) are head n % G of sequence
// seq0 + n / G for n < rows; each row's partial result goes to its own (sequence, head) slot list
// at part `slot`. Otherwise rows = G and the rows are the G heads of sequence s.
template <int CDT, int QDT, int D, int B, bool NT>
__device__ __forceinline__ void mfma_segment(const DecodeArgs& a, float* smem, int s, int g, int L,
                                             int b0, int b1, bool final_out, size_t slot,
                                             int rows, int seq0) {
  constexpr int EB = Elem<CDT>::bytes;
  // Work items: one block (B >= 16: SUB = B/16 tiles of 16 tokens) or, for B = 8, a pair of
  // consecutive blocks forming one 16-token tile (key rows and value token columns 0-7 from the
  // first block, 8-15 from the second).
  static_assert(B == 8 || B == 16 || B == 32, "block size");
  constexpr bool PAIR = B < 16;
  constexpr int GB = PAIR ? 16 / B : 1;      // blocks per work item
  constexpr int SUB = PAIR ? 1 : B / 16;     // 16-token tiles per work item
  constexpr int KK = D / 32;                 // score MFMAs per tile
  constexpr int MI = D / 16;                 // value MFMA tiles (x2 for hi / remainder)
  constexpr int KL = EB == 2 ? KK : KK / 2;  // 16-byte key chunks per lane per tile
  constexpr int KT = 16 * D * EB;            // bytes of one 16-token key tile
  constexpr int KTB = B * D * EB;            // bytes of one (block, kv head) key or value tile
  constexpr int CPR = D * EB / 16;           // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;              // key rows per 1 KB load instruction
  constexpr int NI = 16 / RPI;               // load instructions per key tile
  constexpr int NBI = mfma_blocks_per_iter(EB);  // 16-token tiles per iteration (16 KB in flight)
  constexpr int BPI = NBI / SUB;             // work items per iteration
  constexpr int CHUNK = 64 / GB;             // work items whose table entries one VGPR holds
  static_assert(BPI >= 1 && NBI % SUB == 0, "an iteration takes whole work items");
  constexpr int kKeyAux = NT ? 2 : 0;        // cache policy of the key loads (2: non-temporal)
  constexpr bool kNtV = NT;
  constexpr bool kStageValues = mfma_stages_values(CDT, B);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, n = lane & 15;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  const int nitems = (b1 - b0 + GB - 1) / GB;
  // tokens at or beyond lim belong to a later segment or to no one (the second block of a pair
  // may lie past the segment's end)
  const int lim = min(L, b1 * B);
  // first token of tile u of work item k (relative to the segment)
  auto tile_start = [&](int k, int u) { return (b0 + GB * k) * B + 16 * (u % SUB); };
  // PAIR: the block (0: first, 1: second) holding this lane's tokens 4*q4 .. 4*q4+3 of a tile
  const bool lane_second = PAIR && q4 >= 2;
  // pa_decode_append: the segment holding the unit's last block substitutes the new token
  // (position L-1, row o_new of its tile) for what the cache holds there -- in the staged key
  // tile and in the value registers -- and stores the key row and the value tile rows of its
  // block back (whole lines rather than one element per dim row). A segment whose rows are
  // several sequences' (a group's shared prefix) holds no sequence's own last block.
  const int nblk_all = (L + B - 1) / B;
  const int slot_new = (a.new_slots != nullptr && b1 == nblk_all && rows == G)
                           ? new_token_slot(a, s, L, B) : -1;
  const int item_new = (nblk_all - 1 - b0) / GB;  // (meaningful only when slot_new >= 0)
  const int sub_new = PAIR ? 0 : ((L - 1) % B) / 16;
  const int o_new = (L - 1) - tile_start(item_new, sub_new);

  u32x4 qop[KK];
  if (n < rows) {
    const int sq = seq0 >= 0 ? seq0 + n / G : s;
    const int hq = g * G + (seq0 >= 0 ? n % G : n);
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(a.q) + ((static_cast<size_t>(sq) * Hq + hq) * D) * 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = qp[dim_base<EB>(q4, kk) / 8];
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = u32x4{0u, 0u, 0u, 0u};
  }

  // Key tiles are staged through this wave's NBI LDS slots. Load instruction ii of a tile covers
  // 1 KB of it contiguously (rows RPI*ii .. RPI*ii+RPI-1); lane l fetches 16-byte chunk
  // (l % CPR) ^ (row % CPR) of its row, so LDS holds each row XOR-swizzled by its index and the
  // score-operand reads below (16 rows at one chunk column) fall into distinct banks. PAIR: rows
  // 0-7 come from the first block, 8-15 from the second (dsec: this lane's row is in the second).
  uint8_t* kbuf = reinterpret_cast<uint8_t*>(smem) + wave * (NBI * KT * (kStageValues ? 3 : 1));
  [[maybe_unused]] uint8_t* vbuf = kbuf + 2 * NBI * KT;  // the staged value tiles (kStageValues)
  int dsrc[NI];
  bool dsec[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int row = RPI * ii + lane / CPR;
    dsec[ii] = PAIR && row >= B;
    dsrc[ii] = (dsec[ii] ? row - B : row) * CPR * 16 + 16 * ((lane % CPR) ^ (row % CPR));
  }
  int kread[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) kread[i] = n * CPR * 16 + 16 * ((4 * i + q4) ^ (n % CPR));
  // this lane's value-operand offset inside a block's [D][B] value tile (dim row n, tokens
  // 4*q4 .. 4*q4+3 of the tile), before the tile's token column and the row group mi
  const int vlane = (n * B + 4 * (PAIR ? q4 % 2 : q4)) * EB;

  f32x4 acc[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), lsum = 0.0f;

  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  // this wave's work items are wave + 4*i, taken BPI per iteration (NBI 16-token tiles: tile u is
  // 16-token part u % SUB of item u / SUB); their table entries are fetched CHUNK items at a time
  // into one VGPR (lane GB*j + h: block h of item j) and read back with readlane
  const int nmine = wave < nitems ? (nitems - wave + 3) / 4 : 0;

  // ---- the math of one iteration, shared by both loops below ----
  // scores of the iteration's tiles from the staged keys
  auto tile_scores = [&](const uint8_t* kst, int nlive, f32x4 (&zt)[NBI]) {
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      zt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u / SUB >= nlive) continue;
      const uint8_t* kb = kst + u * KT;
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
  };
  // the online softmax over the iteration's scores: the weights pz, the running max and sum, the
  // accumulator rescaled; valid[u] = this lane group's tokens of tile u below lim (<= 0: none)
  auto online_softmax = [&](int ia, int nlive, const f32x4 (&zt)[NBI], const float (&zs_l)[NBI],
                            int (&valid)[NBI], float (&pz)[4 * NBI]) {
#pragma unroll
    for (int u = 0; u < NBI; ++u)
      valid[u] = u / SUB < nlive ? lim - tile_start(ia + 4 * (u / SUB), u) - 4 * q4 : 0;
    float z[4 * NBI];
#pragma unroll
    for (int u = 0; u < NBI; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[4 * u + i] = (i < valid[u]) ? zt[u][i] * zs_l[u] : neg_inf();
    float tm = z[0];
#pragma unroll
    for (int i = 1; i < 4 * NBI; ++i) tm = fmaxf(tm, z[i]);
    tm = pair32_max(pair16_max(tm));
    const float mn = fmaxf(m, tm);  // finite: the iteration's first item starts below lim
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * NBI; ++i) {
      pz[i] = __builtin_amdgcn_exp2f(z[i] - mn);
      psum += pz[i];
    }
    lsum = lsum * alpha + psum;
    m = mn;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[mi] = acc[mi] * alpha;
  };
  // weighted values, two tiles (32 tokens) per MFMA: k 0..3 are tokens 4*q4.. of the pair's
  // first tile, k 4..7 those of its second; P^T goes in as a 16-bit hi part and remainder.
  // Tokens at or beyond L get zero values (their weights are already 0).
  auto weighted_values = [&](int nlive, const Raw<4 * EB> (&vr)[NBI][MI], const float (&vs_l)[NBI],
                             const float (&pz)[4 * NBI], const int (&valid)[NBI]) {
#pragma unroll
    for (int pr = 0; pr < NBI / 2; ++pr) {
      if ((2 * pr) / SUB >= nlive) break;
      const int u0 = 2 * pr, u1 = 2 * pr + 1;
      // (gfx950's packed converters, round to nearest even: two weights an instruction)
      uint32_t phw[4], plw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = i < 2 ? vs_l[u0] : vs_l[u1];
        const float p0 = pz[4 * u0 + 2 * i] * sc, p1 = pz[4 * u0 + 2 * i + 1] * sc;
        split16x2<QDT>(p0, p1, phw[i], plw[i]);
      }
      const u32x4 phi{phw[0], phw[1], phw[2], phw[3]};
      const u32x4 plo{plw[0], plw[1], plw[2], plw[3]};
      const uint32_t ma0 = valid[u0] >= 2 ? 0xffffffffu : (valid[u0] == 1 ? 0x0000ffffu : 0u);
      const uint32_t ma1 = valid[u0] >= 4 ? 0xffffffffu : (valid[u0] == 3 ? 0x0000ffffu : 0u);
      const uint32_t mb0 = valid[u1] >= 2 ? 0xffffffffu : (valid[u1] == 1 ? 0x0000ffffu : 0u);
      const uint32_t mb1 = valid[u1] >= 4 ? 0xffffffffu : (valid[u1] == 3 ? 0x0000ffffu : 0u);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        uint32_t a0, a1, c0, c1;
        if constexpr (EB == 2) {
          a0 = vr[u0][mi].w[0];
          a1 = vr[u0][mi].w[1];
          c0 = vr[u1][mi].w[0];
          c1 = vr[u1][mi].w[1];
        } else {
          a0 = fp8x2_to16<QDT, false>(vr[u0][mi].w[0]);
          a1 = fp8x2_to16<QDT, true>(vr[u0][mi].w[0]);
          c0 = fp8x2_to16<QDT, false>(vr[u1][mi].w[0]);
          c1 = fp8x2_to16<QDT, true>(vr[u1][mi].w[0]);
        }
        const u32x4 vop{a0 & ma0, a1 & ma1, c0 & mb0, c1 & mb1};
        acc[mi] = mfma_k32<QDT>(vop, phi, acc[mi]);
        acc[mi] = mfma_k32<QDT>(vop, plo, acc[mi]);
      }
    }
  };
  // the table entries of chunk base_i (cnt items) of this wave
  auto chunk_table = [&](int base_i, int cnt) {
    int tv = 0;
    if (lane < cnt * GB) {
      // a pair's second block past the segment's end stands in as its first block: its tokens are
      // masked, but its scales multiply zero weights, so they must be those of a block in use (a
      // free block's may be anything, NaN included)
      const int blk = b0 + GB * (wave + 4 * (base_i + lane / GB)) + lane % GB;
      tv = trow[blk < b1 ? blk : blk - 1];
      tv = tv < 0 ? 0 : (tv >= a.num_blocks ? a.num_blocks - 1 : tv);
    }
    return tv;
  };

  if constexpr (kStageValues) {
  // ---- fp8 keys and values both staged through LDS, each iteration's loads issued one step
  // ahead: the next iteration's keys as soon as this one's keys have landed (they go to the
  // other key slot), its values once this one's value operands are in registers. Every K/V load
  // of the loop is then a direct-to-LDS load whose completion the explicit counts below track;
  // the table entries and the query operands (register loads) are waited for before the first of
  // them. ----
  typedef __attribute__((address_space(4))) const float cfloat_t;  // (scalar loads of the scales)
  constexpr int NVI = KT / 1024;  // value load instructions per tile
  // vmcnt(N) lgkmcnt(0): every direct load but the last N issued, and every LDS access
  constexpr int kWaitKeys = ((NBI * NVI) & 15) | (7 << 4) | (((NBI * NVI) >> 4) << 14);
  constexpr int kWaitValues = ((NBI * NI) & 15) | (7 << 4) | (((NBI * NI) >> 4) << 14);
  constexpr int kWaitLds = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0), no vmcnt wait
  static_assert(NBI * NVI <= 63 && NBI * NI <= 63, "vmcnt field");
  for (int base_i = 0; base_i < nmine; base_i += CHUNK) {
  const int cnt = min(CHUNK, nmine - base_i);
  const int tv = chunk_table(base_i, cnt);
  __builtin_amdgcn_s_waitcnt(0);
  auto tiles_at = [&](int it, int nl, int (&pb)[NBI], size_t (&tb)[NBI]) {
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      pb[u] = __builtin_amdgcn_readlane(tv, it + (u < nl ? u : 0));
      tb[u] = (static_cast<size_t>(pb[u]) * Hkv + g) * KTB;
    }
  };
  auto kslot = [&](int itx) { return kbuf + ((itx / BPI) & 1) * (NBI * KT); };
  auto issue_keys = [&](uint8_t* kdst, int nl, const size_t (&tb)[NBI]) {
#pragma unroll
    for (int u = 0; u < NBI; ++u)
      if (u < nl) {
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) dma16<kKeyAux>(a.k_cache + tb[u] + dsrc[ii], kdst + u * KT + 1024 * ii);
      }
  };
  auto issue_values = [&](int nl, const size_t (&tb)[NBI]) {  // [D][16] codes as stored, 1 KB a load
#pragma unroll
    for (int u = 0; u < NBI; ++u)
      if (u < nl) {
#pragma unroll
        for (int ii = 0; ii < NVI; ++ii)
          dma16<kKeyAux>(a.v_cache + tb[u] + 1024 * ii + 16 * lane, vbuf + u * KT + 1024 * ii);
      }
  };
  auto scales_of = [&](const int (&pb)[NBI], float (&zs)[NBI], float (&vs)[NBI]) {
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      const size_t ix = static_cast<size_t>(pb[u]) * Hkv + g;
      zs[u] = a.zscale * ((cfloat_t*)a.k_scale)[ix];
      vs[u] = ((cfloat_t*)a.v_scale)[ix];
    }
  };
  size_t ba[NBI];
  float zs_l[NBI], vs_l[NBI];
  {
    const int nl = min(BPI, cnt);
    int pba[NBI];
    tiles_at(0, nl, pba, ba);
    issue_keys(kslot(0), nl, ba);
    issue_values(nl, ba);
    scales_of(pba, zs_l, vs_l);
  }
  for (int it = 0; it < cnt; it += BPI) {
    const int nlive = min(BPI, cnt - it);
    const int ia = wave + 4 * (base_i + it);
    const int nl_next = it + BPI < cnt ? min(BPI, cnt - it - BPI) : 0;
    int u_new = -1;
#pragma unroll
    for (int u = 0; u < NBI; ++u)
      if (slot_new >= 0 && u < nlive && ia + 4 * u == item_new) u_new = u;
    // this iteration's keys have landed (its values, issued after them, may still be in flight)
    if (u_new < 0 && nlive == BPI) __builtin_amdgcn_s_waitcnt(kWaitKeys);
    else __builtin_amdgcn_s_waitcnt(0);
    // the next iteration's keys, into the other key slot
    int pba_n[NBI];
    size_t ba_n[NBI];
    float zs_n[NBI], vs_n[NBI];
    if (nl_next > 0) {
      tiles_at(it + BPI, nl_next, pba_n, ba_n);
      issue_keys(kslot(it + BPI), nl_next, ba_n);
      scales_of(pba_n, zs_n, vs_n);
    }
    uint8_t* kcur = kslot(it);
    if (u_new >= 0) {  // the new token's key row into the staged tile and into the cache
      const size_t pbn = static_cast<size_t>(slot_new / B);
      const float ks = a.k_scale[pbn * Hkv + g];
      if (lane < D / 8) {
        const u32x4 kn = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint16_t*>(a.k_new) + (static_cast<size_t>(s) * Hkv + g) * D + 8 * lane);
        Raw<16> in;
        in.w[0] = kn.x; in.w[1] = kn.y; in.w[2] = kn.z; in.w[3] = kn.w;
        const Raw<8> kc = new_key_piece<CDT, QDT, 8>(in, ks);
        store_raw<8>(kcur + u_new * KT + o_new * CPR * 16 + 16 * ((lane / 2) ^ (o_new % CPR)) + 8 * (lane % 2), kc);
        store_raw<8>(const_cast<uint8_t*>(a.k_cache) + (pbn * Hkv + g) * KTB + (slot_new % B) * D + 8 * lane, kc);
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    f32x4 zt[NBI];
    tile_scores(kcur, nlive, zt);
    int valid[NBI];
    float pz[4 * NBI];
    online_softmax(ia, nlive, zt, zs_l, valid, pz);
    // this iteration's values have landed (the next keys, issued after them, may still be in flight)
    if (u_new < 0 && nl_next == BPI) __builtin_amdgcn_s_waitcnt(kWaitValues);
    else __builtin_amdgcn_s_waitcnt(0);
    Raw<4> vr[NBI][MI];  // lane (q4, n): dim row 16*mi + n, tokens 4*q4 .. 4*q4+3 of tile u
#pragma unroll
    for (int u = 0; u < NBI; ++u)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        vr[u][mi].w[0] = *reinterpret_cast<const uint32_t*>(vbuf + u * KT + (16 * mi + n) * 16 + 4 * q4);
    if (u_new >= 0) {  // the new token's value codes into the operands and the block's rows back
      const size_t pbn = static_cast<size_t>(slot_new / B);
      const float vsn = a.v_scale[pbn * Hkv + g];
      const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.v_new) + (static_cast<size_t>(s) * Hkv + g) * D;
#pragma unroll
      for (int u = 0; u < NBI; ++u) {  // (u == u_new: a static index keeps vr in registers)
        if (u != u_new) continue;
        if (o_new >= 4 * q4 && o_new < 4 * q4 + 4) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            put_elem<EB>(vr[u][mi], o_new - 4 * q4, new_value_bits<CDT, QDT>(vn[16 * mi + n], vsn));
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          store_raw<4>(const_cast<uint8_t*>(a.v_cache) + ba[u] + (16 * mi + n) * 16 + 4 * q4, vr[u][mi]);
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    // the value slots are read: the next iteration's values
    if (nl_next > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitLds);
      issue_values(nl_next, ba_n);
    }
    weighted_values(nlive, vr, vs_l, pz, valid);
    if (nl_next > 0) {
#pragma unroll
      for (int u = 0; u < NBI; ++u) {
        ba[u] = ba_n[u];
        zs_l[u] = zs_n[u];
        vs_l[u] = vs_n[u];
      }
    }
  }
  }
  } else {
  for (int base_i = 0; base_i < nmine; base_i += CHUNK) {
  const int cnt = min(CHUNK, nmine - base_i);
  const int tv = chunk_table(base_i, cnt);
  for (int it = 0; it < cnt; it += BPI) {
    const int nlive = min(BPI, cnt - it);  // work items of this iteration (the last may have fewer)
    const int ia = wave + 4 * (base_i + it);  // the iteration's first work item
    // per tile: base of its (first) block's (block, kv head) tiles, of the second block (PAIR)
    size_t ba[NBI], bb[NBI];
    int pba[NBI], pbb[NBI];
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      const int j = it + (u / SUB < nlive ? u / SUB : 0);
      pba[u] = __builtin_amdgcn_readlane(tv, GB * j);
      pbb[u] = PAIR ? __builtin_amdgcn_readlane(tv, GB * j + 1) : pba[u];
      ba[u] = (static_cast<size_t>(pba[u]) * Hkv + g) * KTB;
      bb[u] = (static_cast<size_t>(pbb[u]) * Hkv + g) * KTB;
    }
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      if (u / SUB < nlive) {
#pragma unroll
        for (int ii = 0; ii < NI; ++ii)
          dma16<kKeyAux>(a.k_cache + (dsec[ii] ? bb[u] : ba[u]) + (u % SUB) * KT + dsrc[ii],
                         kbuf + u * KT + 1024 * ii);
      }
    }
    // value tile rows of tile u for this lane: its block, the tile's token column
    size_t vrow[NBI];
#pragma unroll
    for (int u = 0; u < NBI; ++u) vrow[u] = (lane_second ? bb[u] : ba[u]) + (u % SUB) * 16 * EB + vlane;
    Raw<4 * EB> vr[NBI][MI];
#pragma unroll
    for (int u = 0; u < NBI; ++u)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        vr[u][mi] = load_raw<4 * EB, kNtV>(a.v_cache + vrow[u] + 16 * mi * B * EB);
    // the new token's rows, fetched along with the tile they go into (tile u_new of this
    // iteration, if any): lane l < D/8 the key dims 8l .. 8l+7, lane (q4, n) value dims 16*mi + n
    int u_new = -1;
#pragma unroll
    for (int u = 0; u < NBI; ++u)
      if (slot_new >= 0 && u / SUB < nlive && ia + 4 * (u / SUB) == item_new && u % SUB == sub_new)
        u_new = u;
    u32x4 knew{0u, 0u, 0u, 0u};
    uint32_t vnew[MI / 2];  // two 16-bit values a register
    if (u_new >= 0) {
      const size_t row = (static_cast<size_t>(s) * Hkv + g) * D;
      const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.k_new) + row;
      const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.v_new) + row;
      if (lane < D / 8) knew = *reinterpret_cast<const u32x4*>(kn + 8 * lane);
#pragma unroll
      for (int mi = 0; mi < MI; mi += 2)
        vnew[mi / 2] = static_cast<uint32_t>(vn[16 * mi + n]) | (static_cast<uint32_t>(vn[16 * mi + 16 + n]) << 16);
    }

    // key and value scales of the lane's tokens of each tile (fp8; the key scale folded into zscale)
    float zs_l[NBI], vs_l[NBI];
#pragma unroll
    for (int u = 0; u < NBI; ++u) {
      zs_l[u] = a.zscale;
      vs_l[u] = 1.0f;
      if constexpr (CDT == DT_FP8) {
        const size_t ia_s = static_cast<size_t>(pba[u]) * Hkv + g;
        float ks = a.k_scale[ia_s], vsc = a.v_scale[ia_s];
        if constexpr (PAIR) {
          const size_t ib_s = static_cast<size_t>(pbb[u]) * Hkv + g;
          const float ks2 = a.k_scale[ib_s], vs2 = a.v_scale[ib_s];
          ks = lane_second ? ks2 : ks;
          vsc = lane_second ? vs2 : vsc;
        }
        zs_l[u] *= ks;
        vs_l[u] = vsc;
      }
    }
    // The direct-to-LDS loads have landed only once both the vector-memory counter and the LDS
    // counter have drained (waiting on vmcnt alone let the reads below see stale LDS when the
    // staged tile was the last one issued), hence the full wait: vmcnt(0) lgkmcnt(0).
    __builtin_amdgcn_s_waitcnt(0);

    if (u_new >= 0) {
      const size_t pbn = static_cast<size_t>(slot_new / B);  // the new token's block
      float ks = 1.0f, vsn = 1.0f;
      if constexpr (CDT == DT_FP8) {
        ks = a.k_scale[pbn * Hkv + g];
        vsn = a.v_scale[pbn * Hkv + g];
      }
      uint8_t* kslot = const_cast<uint8_t*>(a.k_cache) + (pbn * Hkv + g) * KTB + (slot_new % B) * D * EB;
      uint8_t* krow_lds = kbuf + u_new * KT + o_new * CPR * 16;
      if (lane < D / 8) {  // key row o_new of the staged tile (XOR-swizzled) and of the cache
        Raw<16> in;
        in.w[0] = knew.x; in.w[1] = knew.y; in.w[2] = knew.z; in.w[3] = knew.w;
        const Raw<8 * EB> kc = new_key_piece<CDT, QDT, 8>(in, ks);
        if constexpr (EB == 2) {
          store_raw<16>(krow_lds + 16 * (lane ^ (o_new % CPR)), kc);
          store_raw<16>(kslot + 16 * lane, kc);
        } else {
          store_raw<8>(krow_lds + 16 * ((lane / 2) ^ (o_new % CPR)) + 8 * (lane % 2), kc);
          store_raw<8>(kslot + 8 * lane, kc);
        }
      }
      // value rows: the lanes whose tokens lie in the new token's block store them back
      const bool mine = !PAIR || (lane_second == (o_new >= B));
#pragma unroll
      for (int u = 0; u < NBI; ++u) {  // (u == u_new: a static index keeps vr in registers)
        if (u != u_new) continue;
        if (o_new >= 4 * q4 && o_new < 4 * q4 + 4) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            put_elem<EB>(vr[u][mi], o_new - 4 * q4,
                         new_value_bits<CDT, QDT>((vnew[mi / 2] >> (16 * (mi & 1))) & 0xffffu, vsn));
        }
        if (mine) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            store_raw<4 * EB>(const_cast<uint8_t*>(a.v_cache) + vrow[u] + 16 * mi * B * EB, vr[u][mi]);
        }
      }
    }

    // scores of the iteration's tiles
    f32x4 zt[NBI];
    tile_scores(kbuf, nlive, zt);
    int valid[NBI];
    float pz[4 * NBI];
    online_softmax(ia, nlive, zt, zs_l, valid, pz);
    weighted_values(nlive, vr, vs_l, pz, valid);
  }
  }
  }
  lds_barrier();  // every wave is done with its staged key tiles: the LDS is reused below


  // per-column sum over the four lane groups, then merge the four waves through LDS
  lsum = pair32_sum(pair16_sum(lsum));
  float* sm_m = smem;
  float* sm_l = smem + 64;
  float* sm_o = smem + 128;  // [4 waves][rows][D]
  if (q4 == 0) {
    sm_m[wave * 16 + n] = m;
    sm_l[wave * 16 + n] = lsum;
  }
  if (n < rows) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[(wave * rows + n) * D + 16 * mi + 4 * q4 + i] = acc[mi][i];
  }
  lds_barrier();
  for (int idx = tid; idx < rows * D; idx += 256) {
    const int nn = idx / D, d = idx - (idx / D) * D;
    float M = sm_m[nn];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + nn]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w * 16 + nn];
      const float e = (mw == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      num = __builtin_fmaf(e, sm_o[(w * rows + nn) * D + d], num);
      den = __builtin_fmaf(e, sm_l[w * 16 + nn], den);
    }
    const float o = num / den;
    if (seq0 >= 0) {
      const size_t ix = (static_cast<size_t>(seq0 + nn / G) * Hq + g * G + nn % G) * a.max_parts + slot;
      a.ws_o[ix * D + d] = o;
      if (d == 0) a.ws_ml[ix] = make_float2(M, den);
    } else if (final_out) {
      store_out(a.out, (static_cast<size_t>(s) * Hq + g * G + nn) * D + d, o, a.out_dtype);
    } else {
      a.ws_o[(slot * G + nn) * D + d] = o;
      if (d == 0) a.ws_ml[slot * G + nn] = make_float2(M, den);
    }
  }
  lds_barrier();  // the LDS is free for the next segment
}

// Fixed partitions: one segment per work-group. Grid (kv head, sequence, partition), or with
// a.ordered a 1-D grid of (item, kv head), kv head fastest, over the ordered work list (longest
// work first; see pa_sched.h).
// Launch bounds ask for 3 wave64s per SIMD (at most 168 VGPRs + AGPRs per lane): 2 leaves too
// few tiles in flight per CU, 4 forces spills.
// NT: non-temporal K/V loads (streaming; the default) or cached ones (blocks shared between
// sequences of the batch).
template <int CDT, int QDT, int D, int B, bool NT>
__global__ __launch_bounds__(256, 3) void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int Hq = a.num_heads, G = Hq / a.num_kv_heads;
  int g, s, p, L;
  if (a.ordered) {
    int* lds = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(smem) +
                                      mfma_lds_bytes<CDT, D, B>(G, 0, false));
    g = static_cast<int>(blockIdx.x % a.num_kv_heads);
    const int2 it = ordered_item(a, B, blockIdx.x / a.num_kv_heads, lds);
    if (it.x < 0) return;
    s = __builtin_amdgcn_readfirstlane(it.x);
    p = __builtin_amdgcn_readfirstlane(it.y);
    L = __builtin_amdgcn_readfirstlane(lds[s]);
  } else {
    g = blockIdx.x;
    s = blockIdx.y;
    p = blockIdx.z;
    L = a.lens[s];
    L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  }
  const int nblk = (L + B - 1) / B;
  const int b0 = p * a.part_blocks;
  if (b0 >= nblk) {
    if (p == 0)
      for (int idx = threadIdx.x; idx < G * D; idx += 256)
        store_out(a.out, (static_cast<size_t>(s) * Hq + g * G) * D + idx, 0.0f, a.out_dtype);
    return;
  }
  const int b1 = min(nblk, b0 + a.part_blocks);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  mfma_segment<CDT, QDT, D, B, NT>(a, smem, s, g, L, b0, b1, nparts == 1,
                                (static_cast<size_t>(s) * a.num_kv_heads + g) * a.max_parts + p, G, -1);
}

// Balanced split: work-group i of a.nw takes share i (tiles [share_lo(i), share_lo(i+1)) of the
// flattened (sequence, kv head, block) list, weighted by its place on its CU) and walks it unit by
// unit.
template <int CDT, int QDT, int D, int B, bool NT>
__global__ __launch_bounds__(256, 3) void decode_mfma_balanced_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  constexpr int EB = Elem<CDT>::bytes;
  const size_t stage = mfma_lds_bytes<CDT, D, B>(a.num_heads / a.num_kv_heads, 0, false);
  int* lens_lds = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(smem) + stage);
  int* pref = lens_lds + a.num_seqs;
  scan_batch(a, B, lens_lds, pref);
  const long long hu = a.num_kv_heads;
  const long long W = static_cast<long long>(pref[a.num_seqs]) * hu;
  const int i = blockIdx.x;
  if (i == 0)
    for (int k = threadIdx.x; k <= a.num_seqs; k += blockDim.x) a.ws_pref[k] = pref[k];
  const int nw = balanced_groups(W, a.nw);
  if (i >= nw) return;
  const long long lo = share_lo(W, nw, a.nw_cls, i), hi = share_lo(W, nw, a.nw_cls, i + 1);
  long long t = lo;
  while (t < hi) {
    const int s = find_seq(pref, a.num_seqs, hu, t);
    const int nb = pref[s + 1] - pref[s];
    const long long rel = t - static_cast<long long>(pref[s]) * hu;
    const int g = static_cast<int>(rel / nb);
    const int j = static_cast<int>(rel - static_cast<long long>(g) * nb);
    const long long uend = t - j + nb;
    const long long seg_end = hi < uend ? hi : uend;
    const bool whole = (j == 0) && (seg_end == uend);
    mfma_segment<CDT, QDT, D, B, NT>(a, smem, s, g, lens_lds[s], j, j + static_cast<int>(seg_end - t),
                                  whole, static_cast<size_t>(2 * i + (t == lo ? 0 : 1)), a.num_heads / a.num_kv_heads, -1);
    t = seg_end;
  }
  (void)EB;
}

// pa_decode_grouped: grid (kv head, group or sequence, part). Row y < num_groups: part p of the
// prefix shared by group y -- the members' queries are the rows, so each shared tile is read once
// for all of them. Row num_groups + s: part p of sequence s's own blocks after the prefix. Every
// part is a partial result; the merge kernel combines a sequence's parts (prefix parts first).
// A group's prefix is clamped to the full blocks every member attends, and a sequence's to its
// own full blocks: both kernels take the same value when the prefixes are consistent.
template <int CDT, int QDT, int D, int B, bool NT>
__global__ __launch_bounds__(256, 3) void decode_mfma_grouped_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int g = blockIdx.x, y = blockIdx.y, p = blockIdx.z;
  const int G = a.num_heads / a.num_kv_heads, S = a.num_seqs, pbk = a.part_blocks;
  auto seq_len = [&](int s) {
    const int L = a.lens[s];
    return L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  };
  if (y < a.num_groups) {
    int gs = a.group_start[y], ge = a.group_start[y + 1];
    gs = gs < 0 ? 0 : (gs > S ? S : gs);
    ge = ge < gs ? gs : (ge > S ? S : ge);
    const int m = ge - gs;
    if (m <= 0 || m * G > 16) return;  // (the host checks the group size; trusted data beyond)
    int pbe = a.prefix_blocks[gs];
    for (int k = 0; k < m; ++k) pbe = min(pbe, seq_len(gs + k) / B);
    pbe = pbe < 0 ? 0 : pbe;
    const int b0 = p * pbk, b1 = min(pbe, b0 + pbk);
    if (b0 >= b1) return;
    mfma_segment<CDT, QDT, D, B, NT>(a, smem, gs, g, pbe * B, b0, b1, false, p, m * G, gs);
    return;
  }
  const int s = y - a.num_groups;
  const int L = seq_len(s), nblk = (L + B - 1) / B;
  int pbe = a.prefix_blocks[s];
  pbe = pbe < 0 ? 0 : (pbe > L / B ? L / B : pbe);
  const int p1 = (pbe + pbk - 1) / pbk;
  if (p == 0 && g == 0 && threadIdx.x == 0) a.ws_count[s] = p1 + (nblk - pbe + pbk - 1) / pbk;
  const int b0 = pbe + p * pbk, b1 = min(nblk, b0 + pbk);
  if (b0 >= b1) return;
  mfma_segment<CDT, QDT, D, B, NT>(a, smem, s, g, L, b0, b1, false, p1 + p, G, s);
}

template <int CDT, int QDT, int D, int B>
static hipError_t launch_mfma_dnb(const DecodeArgs& a, hipStream_t st) {
  const int G = a.num_heads / a.num_kv_heads;
  if (a.grouped) {
    // a.max_parts counts a sequence's prefix and own parts together (its slot stride); either kind
    // alone has at most a.max_parts - 1 parts, so the grid's part dimension stops there
    const dim3 grid(a.num_kv_heads, a.num_groups + a.num_seqs, a.max_parts - 1 > 0 ? a.max_parts - 1 : 1);
    const size_t shm = mfma_lds_bytes<CDT, D, B>(16, 0, false);  // up to 16 rows
    if (a.stream_kv) launch_kernel((decode_mfma_grouped_kernel<CDT, QDT, D, B, true>), grid, dim3(256), shm, st, a);
    else launch_kernel((decode_mfma_grouped_kernel<CDT, QDT, D, B, false>), grid, dim3(256), shm, st, a);
    return hipGetLastError();
  }
  const size_t shm = mfma_lds_bytes<CDT, D, B>(G, a.num_seqs, a.balanced != 0);
  if (a.balanced) {
    const dim3 grid(a.nw);
    if (a.stream_kv) launch_kernel((decode_mfma_balanced_kernel<CDT, QDT, D, B, true>), grid, dim3(256), shm, st, a);
    else launch_kernel((decode_mfma_balanced_kernel<CDT, QDT, D, B, false>), grid, dim3(256), shm, st, a);
  } else {
    const dim3 grid = a.ordered ? dim3(a.num_kv_heads * a.num_seqs * a.max_parts)
                                : dim3(a.num_kv_heads, a.num_seqs, a.max_parts);
    const size_t shm_f = mfma_lds_bytes<CDT, D, B>(G, a.num_seqs, a.ordered != 0);
    if (a.stream_kv) launch_kernel((decode_mfma_kernel<CDT, QDT, D, B, true>), grid, dim3(256), shm_f, st, a);
    else launch_kernel((decode_mfma_kernel<CDT, QDT, D, B, false>), grid, dim3(256), shm_f, st, a);
  }
  return hipGetLastError();
}

template <int CDT, int QDT>
static hipError_t launch_mfma_d(const DecodeArgs& a, int D, int B, hipStream_t st) {
  if (D == 64 && B == 8) return launch_mfma_dnb<CDT, QDT, 64, 8>(a, st);
  if (D == 64 && B == 16) return launch_mfma_dnb<CDT, QDT, 64, 16>(a, st);
  if (D == 64 && B == 32) return launch_mfma_dnb<CDT, QDT, 64, 32>(a, st);
  if (D == 128 && B == 8) return launch_mfma_dnb<CDT, QDT, 128, 8>(a, st);
  if (D == 128 && B == 16) return launch_mfma_dnb<CDT, QDT, 128, 16>(a, st);
  if (D == 128 && B == 32) return launch_mfma_dnb<CDT, QDT, 128, 32>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int cdt, int qdt, int D, int B, hipStream_t st) {
  if (cdt == DT_F16 && qdt == DT_F16) return launch_mfma_d<DT_F16, DT_F16>(a, D, B, st);
  if (cdt == DT_BF16 && qdt == DT_BF16) return launch_mfma_d<DT_BF16, DT_BF16>(a, D, B, st);
  if (cdt == DT_FP8 && qdt == DT_F16) return launch_mfma_d<DT_FP8, DT_F16>(a, D, B, st);
  if (cdt == DT_FP8 && qdt == DT_BF16) return launch_mfma_d<DT_FP8, DT_BF16>(a, D, B, st);
  return hipErrorInvalidValue;
}

// Work-groups per CU the balanced kernel keeps resident (from the occupancy calculator): the
// smaller of its two cache-policy instances, so that the plan -- and with it the result bits --
// never depends on the PA_DECODE_SHARED_BLOCKS hint.
int mfma_groups_per_cu(int cdt, int qdt, int D, int B, int G, int S) {
  const void* k[2] = {nullptr, nullptr};
  size_t shm = 0;
#define PA_PICK(C, Q, DD, BB)                                                              \
  if (cdt == C && qdt == Q && D == DD && B == BB) {                                        \
    k[0] = reinterpret_cast<const void*>(&decode_mfma_balanced_kernel<C, Q, DD, BB, true>);  \
    k[1] = reinterpret_cast<const void*>(&decode_mfma_balanced_kernel<C, Q, DD, BB, false>); \
    shm = mfma_lds_bytes<C, DD, BB>(G, S, true);                                           \
  }
#define PA_PICK_B(C, Q, DD) PA_PICK(C, Q, DD, 8) PA_PICK(C, Q, DD, 16) PA_PICK(C, Q, DD, 32)
  PA_PICK_B(DT_F16, DT_F16, 64) PA_PICK_B(DT_F16, DT_F16, 128) PA_PICK_B(DT_BF16, DT_BF16, 64)
  PA_PICK_B(DT_BF16, DT_BF16, 128) PA_PICK_B(DT_FP8, DT_F16, 64) PA_PICK_B(DT_FP8, DT_F16, 128)
  PA_PICK_B(DT_FP8, DT_BF16, 64) PA_PICK_B(DT_FP8, DT_BF16, 128)
#undef PA_PICK_B
#undef PA_PICK
  if (k[0] == nullptr) return 0;
  int best = 0;
  for (int i = 0; i < 2; ++i) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k[i], 256, shm) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    best = i == 0 ? n : (n < best ? n : best);
  }
  return best;
}

}  // namespace pa
