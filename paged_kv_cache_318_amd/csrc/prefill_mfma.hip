// Causal paged attention of a chunk of new query tokens per sequence (prefill of the chunk over
// the cached context) on gfx950 matrix cores.
//
// The equations of "PagedAttention" (Wikipedia article, section "Математическая формулировка")
// hold for any query position i: query token i attends the keys at positions 1..i, read block by
// block through the table, the last block cut at i. A chunk of n new tokens of a sequence holding
// L tokens (the chunk's keys and values already written) has queries at positions L-n .. L-1.
//
// Rows: the n * G (query token, query head of the kv group) pairs of one (sequence, kv head),
// token-major. One work-group (4 wave64s) takes 128 consecutive rows (64 for fp8 at D = 128);
// each wave takes two sets of 16 (one), each set the 16 columns of the same 16x16x32 MFMA the
// decode kernel uses:
//     Z^T[16 tokens][16 rows]  = K_tile[16][D] . Q^T[D][16 rows]        (scores)
//     O^T[D][16 rows]         += V^T[D][32 tokens] . P^T[32 tokens][16 rows]
// so every K/V tile is fetched once per 128 rows, and every key or value operand read from LDS
// feeds both sets. Per iteration the work-group stages two 16-token key and value tiles (16 KB at
// 16 bits) in LDS with gfx950's direct global -> LDS loads (1 KB contiguous per load
// instruction; keys XOR-swizzled by row so the MFMA-layout reads hit distinct banks), then every
// wave runs its scores, its online softmax and its weighted values out of LDS. Each column
// carries its own causal limit (its query position); a wave's rows never leave it, so no
// cross-wave merge is needed and no workspace either.

#include <climits>
#include <type_traits>

#include "mfma_common.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Column sets per wave: each wave takes CW sets of 16 rows, so every key or value operand read
// from LDS feeds CW MFMAs (one per set). Two sets halve the LDS reads, the K/V fetches and the
// barriers per row; the fp8 instances at D = 128 keep one (their converted operands would spill).
template <int CDT, int D>
constexpr int prefill_column_sets() { return (CDT == DT_FP8 && D == 128) ? 1 : 2; }
template <int CDT, int D>
constexpr int prefill_rows() { return 64 * prefill_column_sets<CDT, D>(); }  // rows per work-group

// Iterations in flight: a ring of this many LDS buffers, so the loads of the next NS-1
// iterations fly while one computes. 2, 3 and 4 stages measured the same (the loop is bound by
// its own issue and latency, not by the loads), so the ring stays at the smallest.
constexpr int kPrefillStages = 2;

// Bytes of one stage: the key tiles of an iteration's two 16-token tiles, their value tiles and,
// for fp8 caches, 256 bytes whose first 32 hold the key and value scales of its (up to 4) blocks.
template <int CDT, int D>
constexpr size_t prefill_stage_bytes() {
  return size_t{4} * 16 * D * Elem<CDT>::bytes + (CDT == DT_FP8 ? 256 : 0);
}

template <int CDT, int D>
constexpr size_t prefill_lds_bytes() {
  return size_t{kPrefillStages} * prefill_stage_bytes<CDT, D>();
}

// The sequence of rank r when the num_seqs sequences are ordered by length, longest first (ties:
// lower index first). Lane j of the wave ranks sequences j, j + 64, ...: every work-group
// computes the same permutation from the lengths alone. Past 256 sequences the order is the
// sequences' own (the ranking would cost more than it saves).
__device__ int seq_by_length_rank(const int32_t* lens, int S, int r, int lane, int maxL) {
  if (S > 256) return r;
  for (int j0 = 0; j0 < S; j0 += 64) {
    const int j = j0 + lane;
    const int kj = j < S ? min(max(lens[j], 0), maxL) : -1;
    int rank = 0;
    for (int i0 = 0; i0 < S; i0 += 64) {
      const int ki_l = i0 + lane < S ? min(max(lens[i0 + lane], 0), maxL) : -1;
      const int n = min(64, S - i0);
      for (int t = 0; t < n; ++t) {
        const int ki = __builtin_amdgcn_readlane(ki_l, t);
        rank += (ki > kj || (ki == kj && i0 + t < j)) ? 1 : 0;
      }
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(j < S && rank == r);
    if (hit != 0) return j0 + static_cast<int>(__builtin_ctzll(hit));
  }
  return r;  // not reached: the ranks are a permutation of 0 .. S-1
}

// Three wave64s per SIMD (at most 168 registers a lane): the two-column-set instances at D = 128
// need a few more, and the compiler spills 4 or 5 of them around the second loop, never inside
// either loop (two waves per SIMD with no spill ran 5% slower).
template <int CDT, int QDT, int D, int B>
__global__ __launch_bounds__(256, 3) void prefill_mfma_kernel(PrefillArgs a) {
  static_assert(B == 8 || B == 16 || B == 32, "block size");
  constexpr int NBL = 32 / B;                // blocks an iteration (32 tokens) touches
  constexpr int CW = prefill_column_sets<CDT, D>();
  constexpr int ROWS = prefill_rows<CDT, D>();
  constexpr int EB = Elem<CDT>::bytes;
  constexpr int KK = D / 32;                 // score MFMAs per 16-token tile
  constexpr int MI = D / 16;                 // value MFMA tiles (x2 for bf16 hi / remainder)
  // The weights P reach the value MFMA as 16-bit operands: fp16 weights keep 11 significant bits,
  // enough for the 2e-3 tolerance, and go as one operand; bf16 weights (8 bits) go as a rounded
  // part plus its remainder, two MFMAs.
  constexpr bool kSplitP = QDT == DT_BF16;
  constexpr int KL = EB == 2 ? KK : KK / 2;  // 16-byte key chunks per lane per tile
  constexpr int KT = 16 * D * EB;            // bytes of one 16-token key (or value) tile in LDS
  constexpr int KTB = B * D * EB;            // bytes of one (block, kv head) tile in the cache
  constexpr int CPR = D * EB / 16;           // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;              // key rows per 1 KB load
  constexpr int NCH = KT / 1024;             // 1 KB loads per tile
  static_assert(NCH >= 1 && KT % 1024 == 0, "tile must be a whole number of 1 KB loads");
  constexpr int NS = kPrefillStages;
  constexpr int SB = static_cast<int>(prefill_stage_bytes<CDT, D>());
  // vector-memory operations one issue() makes per wave: its 1 KB loads, plus (fp8) the load of
  // scales of the iteration's blocks
  constexpr int OPS = NCH + (CDT == DT_FP8 ? 1 : 0);
  static_assert((NS - 2) * OPS <= 63, "vmcnt field");
  // vmcnt((NS-2)*OPS) lgkmcnt(0): every load but those of the NS-2 iterations issued after
  // this one, and every LDS access
  constexpr int kWaitOldest = (((NS - 2) * OPS) & 15) | (7 << 4) | ((((NS - 2) * OPS) >> 4) << 14);
  extern __shared__ float smem[];
  // [NS stages][keys of tiles A, B][values of tiles A, B (dim-major)][fp8 scales]
  uint8_t* kt = reinterpret_cast<uint8_t*>(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, q4 = lane >> 4, n = lane & 15;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
  // Work-group order (the hardware starts work-groups in index order): sequences longest first,
  // each one's row tiles from the last (whose queries attend the most tokens) to the first, kv
  // heads innermost. The longest work-groups start first and short ones fill the tail; with 8 kv
  // heads, the tiles of one (sequence, kv head) all land on the same XCD and share its L2.
  const int wg = blockIdx.x;
  const int g = wg % Hkv;
  const int tile = a.num_tiles - 1 - (wg / Hkv) % a.num_tiles;
  const int s = seq_by_length_rank(a.lens, a.num_seqs, wg / Hkv / a.num_tiles, lane, a.max_blocks * B);

  int L = a.lens[s];
  L = L < 0 ? 0 : (L > a.max_blocks * B ? a.max_blocks * B : L);
  int q0 = a.query_start[s], q1 = a.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.num_tokens ? a.num_tokens : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.num_tokens ? a.num_tokens : q1);
  const int ns = (q1 - q0) < L ? (q1 - q0) : L;  // a chunk cannot be longer than the sequence
  const int rows = ns * G;
  const int r0 = tile * ROWS;
  if (r0 >= rows) return;
  const int rlast = (r0 + ROWS < rows ? r0 + ROWS : rows) - 1;
  const int ntok = L - ns + rlast / G + 1;         // tokens up to the group's last query
  const int nblk = (ntok + B - 1) / B;

  // this lane's columns: row r = (token k of the chunk, head hh of the group) of set c; rows past
  // the chunk attend token 0 only (finite, discarded)
  const int wrow = r0 + wave * 16 * CW;
  bool live[CW];
  int kq[CW], hh[CW], pos[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const int r = wrow + 16 * c + n;
    live[c] = r < rows;
    kq[c] = live[c] ? r / G : 0;
    hh[c] = live[c] ? r - kq[c] * G : 0;
    pos[c] = live[c] ? L - ns + kq[c] : 0;
  }
  // earliest query position among the wave's columns (0 if the wave has rows past the chunk,
  // which attend token 0 only)
  const int wave_min_pos = wrow + 16 * CW - 1 < rows ? L - ns + wrow / G : 0;


  // Load c (c = wave + 4*i) of the iteration's 4*NCH 1 KB loads: c < 2*NCH are keys (tile
  // c / NCH, part c % NCH of it), the rest values. An iteration covers 32 tokens: tile A (tokens
  // 0-15) and tile B (16-31), read from the NBL blocks they lie in; each lane's 16-byte piece
  // comes from block ld_blk of the iteration, at offset ld_src inside that block's tile.
  // LDS stage: keys of tiles A and B ([2][KT], rows XOR-swizzled), then their values. 16-bit
  // values are stored per 16-row group mi as 1 KB: [tile A, B][half][row] of 16-byte halves (8
  // tokens) of the [row][16 tokens] rows. The value-operand read of lane (q4, n) (row n, tokens
  // 4*q4 .. 4*q4+3) then covers 512 contiguous bytes per tile, each 8-byte piece once (no bank
  // conflicts; the [row][half] order would put rows n and n+8 on the same banks), and its two
  // 8-byte pieces (tile A, tile B) sit 512 bytes apart: one paired read fills the operand.
  // fp8 values: [row][16 tokens] per tile (16-byte rows read without conflicts); at B = 8 a
  // tile's 16 tokens span two blocks, so each block's [D][8] tile is staged as it is stored
  // ([half][row][8 tokens]: a 16-byte piece is two consecutive rows of one block).
  // Value loads: 16-bit, group mi = c - 2*NCH, lanes 0-31 tile A, 32-63 tile B; fp8, tile
  // (c - 2*NCH) / NCH, part (c - 2*NCH) % NCH.
  int ld_dst[NCH], ld_src[NCH], ld_blk[NCH];
  bool ld_key[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = wave + 4 * i;
    ld_key[i] = c < 2 * NCH;
    if (c < 2 * NCH) {  // keys: lane fetches chunk (lane % CPR) ^ (row % CPR) of its row
      const int t = c / NCH, part = c % NCH;
      const int row = RPI * part + lane / CPR;
      const int tok = 16 * t + row;
      ld_blk[i] = tok / B;
      ld_src[i] = (tok % B) * CPR * 16 + 16 * ((lane % CPR) ^ (row % CPR));
      ld_dst[i] = t * KT + 1024 * part;
    } else if constexpr (EB == 2) {
      const int mi = c - 2 * NCH, t = lane / 32, hf = (lane % 32) / 16, row = 16 * mi + lane % 16;
      const int tok = 16 * t + 8 * hf;
      ld_blk[i] = tok / B;
      ld_src[i] = (row * B + tok % B) * EB;
      ld_dst[i] = 2 * KT + 1024 * mi;
    } else {
      const int v = c - 2 * NCH, t = v / NCH, part = v % NCH;
      ld_dst[i] = 2 * KT + t * KT + 1024 * part;
      if constexpr (B >= 16) {
        const int row = part * 64 + lane;
        ld_blk[i] = (16 * t) / B;
        ld_src[i] = row * B + (16 * t) % B;
      } else {
        const int q = part * 1024 + 16 * lane;  // byte of the tile's [half][row][8] stage
        ld_blk[i] = 2 * t + q / (8 * D);
        ld_src[i] = q % (8 * D);
      }
    }
  }
  int kread[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) kread[i] = n * CPR * 16 + 16 * ((4 * i + q4) ^ (n % CPR));

  f32x4 acc[CW][MI];
  float m[CW], lsum[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[c][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = neg_inf();
    lsum[c] = 0.0f;
  }

  // Iteration i covers tokens 32i .. 32i+31 (tile B may lie past the group's last query).
  // Its tiles go to LDS buffer i % NS: the loads for i+NS-1 are issued right after the barrier
  // that opens iteration i (every wave is then done with buffer (i-1) % NS), so NS-1 iterations
  // of loads fly while iteration i computes.
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const int niter = (ntok + 31) / 32;
  int tv = 0, tbase = -64;
  auto issue = [&](int it) {
    const int jb0 = NBL * it;  // the iteration's first block
    if (jb0 - tbase >= 64) {  // next 64 table entries into one VGPR, read back with readlane
      tbase = jb0;
      tv = 0;
      if (tbase + lane < nblk) {
        tv = trow[tbase + lane];
        tv = tv < 0 ? 0 : (tv >= a.num_blocks ? a.num_blocks - 1 : tv);
      }
    }
    // blocks past the group's last query stand in as the iteration's first: their tokens are
    // masked, but their scales multiply zero weights, so they must be those of a block in use
    int pb[NBL];
    pb[0] = __builtin_amdgcn_readlane(tv, jb0 - tbase);
#pragma unroll
    for (int k = 1; k < NBL; ++k)
      pb[k] = jb0 + k < nblk ? __builtin_amdgcn_readlane(tv, jb0 + k - tbase) : pb[0];
    uint8_t* buf = kt + (it % NS) * SB;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int p = pb[0];
#pragma unroll
      for (int k = 1; k < NBL; ++k) p = ld_blk[i] == k ? pb[k] : p;
      const uint8_t* src = (ld_key[i] ? a.k_cache : a.v_cache) +
                           (static_cast<size_t>(p) * Hkv + g) * KTB + ld_src[i];
      dma16<0>(src, buf + ld_dst[i]);
    }
    if constexpr (CDT == DT_FP8) {
      // 4 bytes a lane into the stage's scale slot: lane l holds the key scale of block l % 8
      // for l % 8 < NBL, the value scale of block l % 8 - 4 for 4 <= l % 8 < 4 + NBL (every wave
      // writes the same values; each issues it, so all count the same loads)
      const int w8 = lane % 8, k = w8 % 4;
      int p = pb[0];
#pragma unroll
      for (int kk = 1; kk < NBL; ++kk) p = (k < NBL && k == kk) ? pb[kk] : p;
      const float* sp = w8 >= 4 ? a.v_scale : a.k_scale;
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(sp + static_cast<size_t>(p) * Hkv + g),
                                       (lds_void_t*)(buf + 4 * KT), 4, 0, 0);
    }
  };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < niter) issue(j);
  // the query operands, loaded behind the first tiles; then one full wait, so that the loop
  // starts with nothing in flight but what its own waits account for
  u32x4 qop[CW][KK];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    if (live[c]) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          reinterpret_cast<const uint8_t*>(a.q) +
          ((static_cast<size_t>(q0 + kq[c]) * Hq + g * G + hh[c]) * D) * 2);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qop[c][kk] = qp[dim_base<EB>(q4, kk) / 8];
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qop[c][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  // 16-bit caches scale every score by one factor, zsp = |scale * log2(e)|: a negative scale
  // goes into the query's sign bits (exact), so that the running max can be taken on the
  // unscaled scores and the factor applied inside the exponent's FMA
  const float zsp = EB == 2 ? fabsf(a.zscale) : a.zscale;
  if constexpr (EB == 2) {
    if (a.zscale < 0.0f) {
#pragma unroll
      for (int c = 0; c < CW; ++c)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          qop[c][kk] = u32x4{qop[c][kk].x ^ 0x80008000u, qop[c][kk].y ^ 0x80008000u,
                             qop[c][kk].z ^ 0x80008000u, qop[c][kk].w ^ 0x80008000u};
    }
  }
  auto body = [&](const int it, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int t0a = 32 * it;           // first token of tile A
    const bool has_b = t0a + 16 < ntok;
    const int slot = it % NS;
    // This wave's loads for iteration it have landed: the vector-memory counter is down to the
    // loads of the iterations issued after it (all of them near the end, when fewer are left)
    // and the LDS counter has drained. After the barrier every wave's have, and every wave is
    // done reading buffer (it-1) % NS, which the loads issued below go to.
    // The barrier is a bare s_barrier behind these explicit waits (the compiler's own barrier
    // lowering waits for every load in flight, which would drain the ring each iteration); the
    // empty asm statements keep the compiler from moving memory accesses across it.
    if (it + NS - 2 < niter) __builtin_amdgcn_s_waitcnt(kWaitOldest);
    else __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint8_t* kb0 = kt + slot * SB;
    const uint8_t* vt = kb0 + 2 * KT;
    // key and value scales of this lane's tokens of tiles A and B (block (16u + 4*q4) / B)
    float zs[2] = {zsp, zsp}, vs[2] = {1.0f, 1.0f};
    if constexpr (CDT == DT_FP8) {
      const float* scl = reinterpret_cast<const float*>(kb0 + 4 * KT);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int bi = (16 * u + 4 * q4) / B;
        zs[u] *= scl[bi];
        vs[u] = scl[4 + bi];
      }
    }
    if (it + NS - 1 < niter) issue(it + NS - 1);

    // scores: each key operand read once from LDS, multiplied into every column set
    f32x4 zt[CW][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int c = 0; c < CW; ++c) zt[c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kb = kb0 + u * KT;
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(kb + kread[i]);
        if constexpr (EB == 2) {
#pragma unroll
          for (int c = 0; c < CW; ++c) zt[c][u] = mfma_k32<QDT>(raw, qop[c][i], zt[c][u]);
        } else {
          const u32x4 k0{fp8x2_to16<QDT, false>(raw.x), fp8x2_to16<QDT, true>(raw.x),
                         fp8x2_to16<QDT, false>(raw.y), fp8x2_to16<QDT, true>(raw.y)};
          const u32x4 k1{fp8x2_to16<QDT, false>(raw.z), fp8x2_to16<QDT, true>(raw.z),
                         fp8x2_to16<QDT, false>(raw.w), fp8x2_to16<QDT, true>(raw.w)};
#pragma unroll
          for (int c = 0; c < CW; ++c) {
            zt[c][u] = mfma_k32<QDT>(k0, qop[c][2 * i], zt[c][u]);
            zt[c][u] = mfma_k32<QDT>(k1, qop[c][2 * i + 1], zt[c][u]);
          }
        }
      }
    }
    // per column set: online softmax of lane (q4, n)'s tokens t0(u) .. t0(u)+3 of tile u
    u32x4 phi[CW], plo[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      // z: the scores of lane (q4, n)'s tokens, unscaled for 16-bit caches (one common factor
      // zsp >= 0, applied in the exponent), scaled per tile for fp8; ok: inside the causal
      // limit and (tile B) inside the group's tokens
      float z[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t0 = t0a + 16 * u + 4 * q4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ok[4 * u + i] = !MASKED || (t0 + i <= pos[c] && (u == 0 || has_b));
          z[4 * u + i] = EB == 2 ? zt[c][u][i] : zt[c][u][i] * zs[u];
        }
      }
      // The accumulators are rescaled to a new running max only when some column of the set
      // sees a score above its max by more than kSlack (log2 units); until then its weights run
      // up to 2^kSlack (the result is the same for any common shift, the final division takes
      // it out). bf16 has fp32's range and fp16 holds 2^8; only fp16 weights times an fp8 value
      // scale keep the eager rescale, so that their product cannot overflow.
      constexpr float kSlack = (QDT == DT_BF16 || CDT != DT_FP8) ? 8.0f : 0.0f;
      // weights of the lane's 8 tokens from the running max as it stands, and their sum
      float pz[8];
      auto weights = [&]() {
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = EB == 2 ? __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], zsp, -m[c]))
                                  : __builtin_amdgcn_exp2f(z[i] - m[c]);
          pz[i] = ok[i] ? e : 0.0f;
          ps += pz[i];
        }
        return ps;
      };
      // the columns' max over the iteration's tokens, and the rescale if some column needs it
      // (returns whether it rescaled)
      auto rescale = [&]() {
        float zm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) zm[i] = ok[i] ? z[i] : neg_inf();
        // a chain, which the compiler folds into 3-input maxes
        float tm = zm[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tm = fmaxf(tm, zm[i]);
        tm = pair32_max(pair16_max(tm));
        // -inf * 0 (every token of a column masked, zero scale) is NaN: compares false below
        if constexpr (EB == 2) tm *= zsp;
        if (__builtin_amdgcn_ballot_w64(tm > m[c] + kSlack) == 0) return false;
        const float mn = fmaxf(m[c], tm);  // finite: block 0 holds token 0, which every column attends
        const float alpha = __builtin_amdgcn_exp2f(m[c] - mn);
        lsum[c] *= alpha;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) acc[c][mi] = acc[c][mi] * alpha;
        m[c] = mn;
        return true;
      };
      float ps;
      if constexpr (kSlack > 0.0f) {
        // Weights first: while every lane's 8 weights sum to at most 2^kSlack (so each is at
        // most that), the max is not needed at all. Otherwise (a large score, the first
        // iteration's -inf max, or inf / NaN) the max decides, and the weights are taken again
        // if it moved.
        ps = weights();
        if (__builtin_amdgcn_ballot_w64(!(ps <= __builtin_exp2f(kSlack))) != 0 && rescale())
          ps = weights();
      } else {
        rescale();
        ps = weights();
      }
      lsum[c] += ps;
      // P^T: one fp16 operand, or bf16 hi part + remainder
      uint32_t phw[4], plw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float vsc = i < 2 ? vs[0] : vs[1];
        const float p0 = pz[2 * i] * vsc, p1 = pz[2 * i + 1] * vsc;
        if constexpr (kSplitP) split16x2<QDT>(p0, p1, phw[i], plw[i]);
        else phw[i] = pack16x2<QDT>(p0, p1);
      }
      phi[c] = u32x4{phw[0], phw[1], phw[2], phw[3]};
      if constexpr (kSplitP) plo[c] = u32x4{plw[0], plw[1], plw[2], plw[3]};
    }
    // weighted values over the 32 tokens of the two tiles; slots at or beyond L (never
    // written) get zero values
    uint32_t ma0 = ~0u, ma1 = ~0u, mb0 = ~0u, mb1 = ~0u;
    if constexpr (MASKED) {
      const int va = L - t0a - 4 * q4;                      // this lane group's tokens below L
      const int vb = has_b ? L - t0a - 16 - 4 * q4 : 0;
      ma0 = va >= 2 ? 0xffffffffu : (va == 1 ? 0x0000ffffu : 0u);
      ma1 = va >= 4 ? 0xffffffffu : (va == 3 ? 0x0000ffffu : 0u);
      mb0 = vb >= 2 ? 0xffffffffu : (vb == 1 ? 0x0000ffffu : 0u);
      mb1 = vb >= 4 ? 0xffffffffu : (vb == 3 ? 0x0000ffffu : 0u);
    }
    // value operand of group mi: tokens 4*q4 .. 4*q4+3 of tile A, then of tile B
    auto vop_of = [&](int mi) -> u32x4 {
      uint32_t a0, a1, c0, c1;
      if constexpr (EB == 2) {
        const int voff = 1024 * mi + 256 * (q4 / 2) + 16 * n + 8 * (q4 % 2);
        const u32x2 x = *reinterpret_cast<const u32x2*>(vt + voff);
        const u32x2 y = *reinterpret_cast<const u32x2*>(vt + voff + 512);
        a0 = x.x;
        a1 = x.y;
        c0 = y.x;
        c1 = y.y;
      } else {
        const int voff = B >= 16 ? (16 * mi + n) * 16 + 4 * q4
                                 : (q4 / 2) * (8 * D) + (16 * mi + n) * 8 + 4 * (q4 % 2);
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vt + voff);
        const uint32_t y = *reinterpret_cast<const uint32_t*>(vt + KT + voff);
        a0 = fp8x2_to16<QDT, false>(x);
        a1 = fp8x2_to16<QDT, true>(x);
        c0 = fp8x2_to16<QDT, false>(y);
        c1 = fp8x2_to16<QDT, true>(y);
      }
      if constexpr (MASKED) return u32x4{a0 & ma0, a1 & ma1, c0 & mb0, c1 & mb1};
      else return u32x4{a0, a1, c0, c1};
    };
    // each value operand read once from LDS and multiplied into every column set; groups of
    // 4 value tiles (for bf16, hi MFMAs of the group, then its remainder MFMAs) so no MFMA waits
    // on the one just issued into the same accumulator
    constexpr int GV = CW == 1 ? 4 : 2;
#pragma unroll
    for (int m0 = 0; m0 < MI; m0 += GV) {
      u32x4 vop[GV];
#pragma unroll
      for (int j = 0; j < GV; ++j) {
        vop[j] = vop_of(m0 + j);
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[c][m0 + j] = mfma_k32<QDT>(vop[j], phi[c], acc[c][m0 + j]);
      }
      if constexpr (kSplitP) {
#pragma unroll
        for (int j = 0; j < GV; ++j)
#pragma unroll
          for (int c = 0; c < CW; ++c) acc[c][m0 + j] = mfma_k32<QDT>(vop[j], plo[c], acc[c][m0 + j]);
      }
    }
  };
  // Interior iterations (every token of both tiles at or before the wave's earliest query, so
  // also below L) need neither the causal nor the end-of-sequence mask; they come first and run
  // in a loop of their own. With both kinds in one loop the compiler gave the accumulators
  // different registers on the two paths and copied all of them every iteration.
  const int n_interior = min((wave_min_pos + 1) / 32, niter);
  int it = 0;
  for (; it < n_interior; ++it) body(it, std::false_type{});
  for (; it < niter; ++it) body(it, std::true_type{});

#pragma unroll
  for (int c = 0; c < CW; ++c) {
    float ls = lsum[c];
    ls = pair32_sum(pair16_sum(ls));
    if (live[c]) {
      const size_t orow = (static_cast<size_t>(q0 + kq[c]) * Hq + g * G + hh[c]) * D;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const f32x4 o{acc[c][mi][0] / ls, acc[c][mi][1] / ls, acc[c][mi][2] / ls, acc[c][mi][3] / ls};
        store_out4(a.out, orow + 16 * mi + 4 * q4, o, a.out_dtype);
      }
    }
  }
}

template <int CDT, int QDT, int D, int B>
static hipError_t launch_prefill_dnb(const PrefillArgs& a, int max_query_len, hipStream_t st) {
  const int G = a.num_heads / a.num_kv_heads;
  const long long rows = static_cast<long long>(max_query_len) * G;
  constexpr int R = prefill_rows<CDT, D>();
  PrefillArgs args = a;
  const long long tiles = (rows + R - 1) / R;
  const long long wgs = tiles * a.num_kv_heads * a.num_seqs;  // one-dimensional grid
  if (tiles > INT_MAX || wgs > INT_MAX) return hipErrorInvalidValue;
  args.num_tiles = static_cast<int>(tiles);
  const size_t shm = prefill_lds_bytes<CDT, D>();
  launch_kernel((prefill_mfma_kernel<CDT, QDT, D, B>), dim3(static_cast<unsigned>(wgs)),
                     dim3(256), shm, st, args);
  return hipGetLastError();
}

template <int CDT, int QDT, int D>
static hipError_t launch_prefill_dn(const PrefillArgs& a, int B, int max_query_len, hipStream_t st) {
  if (B == 8) return launch_prefill_dnb<CDT, QDT, D, 8>(a, max_query_len, st);
  if (B == 16) return launch_prefill_dnb<CDT, QDT, D, 16>(a, max_query_len, st);
  if (B == 32) return launch_prefill_dnb<CDT, QDT, D, 32>(a, max_query_len, st);
  return hipErrorInvalidValue;
}

template <int CDT, int QDT>
static hipError_t launch_prefill_d(const PrefillArgs& a, int D, int B, int max_query_len, hipStream_t st) {
  if (D == 64) return launch_prefill_dn<CDT, QDT, 64>(a, B, max_query_len, st);
  if (D == 128) return launch_prefill_dn<CDT, QDT, 128>(a, B, max_query_len, st);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, int cdt, int qdt, int D, int B, int max_query_len,
                          hipStream_t st) {
  if (cdt == DT_F16 && qdt == DT_F16) return launch_prefill_d<DT_F16, DT_F16>(a, D, B, max_query_len, st);
  if (cdt == DT_BF16 && qdt == DT_BF16) return launch_prefill_d<DT_BF16, DT_BF16>(a, D, B, max_query_len, st);
  if (cdt == DT_FP8 && qdt == DT_F16) return launch_prefill_d<DT_FP8, DT_F16>(a, D, B, max_query_len, st);
  if (cdt == DT_FP8 && qdt == DT_BF16) return launch_prefill_d<DT_FP8, DT_BF16>(a, D, B, max_query_len, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
