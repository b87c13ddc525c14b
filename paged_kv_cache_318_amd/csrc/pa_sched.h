// Work order of the decode kernels (device side): the balanced split, and the ordered work list
// of fixed partitions (further below).
//
// Balanced split. The batch's work is the flattened list of (sequence, unit, block) tiles,
// sequence-major: a "unit" is what one work-group accumulates (a query head for the VALU kernel, a
// kv head with its query group for the MFMA kernel), and unit (s, x) owns nblk(s) consecutive
// tiles. With W tiles in all and nw work-groups, work-group i takes tiles
// [share_lo(i), share_lo(i+1)): equal shares, or, on a resident grid of three work-groups per CU
// with long shares, shares weighted by the work-group's order of arrival on its CU (below), so
// that the work-groups finish together whatever the length mix. A unit cut by a share boundary is
// finished by the merge kernel from the partial results of the work-groups that share it (at most
// two partial results per work-group: its first and its last unit), combined with the same
// log-sum-exp algebra as the rest of the method.
//
// Every work-group recomputes the prefix sums of the block counts in LDS from the lengths (no
// extra launch); work-group 0 also leaves them in the workspace for the merge kernel. The grid
// launched is an upper bound: only the first balanced_groups(W, nw) work-groups take a share,
// which keeps every share at least kMinShareTiles tiles long (never empty) however short the
// batch.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kMaxBalancedSeqs = 1024;    // batches up to this many sequences use the split
constexpr int kMaxBalancedGroups = 2048;  // grid bound (sizes the partial-result workspace)

constexpr int kMinShareTiles = 16;        // one iteration of two blocks for each of 4 waves, twice

// Work-groups that take a share of W tiles when nw are launched: between 1 and nw.
__device__ __forceinline__ int balanced_groups(long long W, int nw) {
  const long long n = W / kMinShareTiles;
  return n < 1 ? 1 : (n > nw ? nw : static_cast<int>(n));
}

// Shares weighted by the work-group's place on its CU. The resident grid is dispatched one
// work-group per CU at a time, so with cls CUs and three work-groups per CU, work-group i is the
// (i / cls)-th to arrive on its CU. The three do not progress at the same rate: the CU favours its
// older waves, and with equal shares the first, second and third to arrive finished after ~94, ~104
// and ~134 us (16 fp8 sequences of 16K..32K tokens), the last third running alone on its CU at about
// two thirds of the CU's rate. Shares in the proportion 28 : 20 : 12 bring the three close to
// finishing together: that batch's kernel took 135.2 us, against 149.1 with equal shares, 144.3 at
// 24 : 20 : 16, 138.4 at 26 : 20 : 14 and 140.5 at 30 : 20 : 10. The shares depend only on the batch
// and the CU count, so results stay deterministic.
// Short shares are not bandwidth-shared long enough for the order to matter, and the heavier
// first shares then only lengthen the critical path (16 GQA sequences, about 17 bf16 tiles a share:
// 35.2 us weighted against 28.4 us equal; 4 fp8 sequences, 64 tiles a share: 47.0 against 51.6):
// the weights apply from kWeightedMinTiles tiles a share on average.
constexpr int kSlotWeight0 = 28, kSlotWeight1 = 20, kSlotWeight2 = 12;
constexpr int kSlotWeightSum = kSlotWeight0 + kSlotWeight1 + kSlotWeight2;
constexpr int kWeightedMinTiles = 48;

// Whether a grid of nw shares over W tiles is the weighted one.
__device__ __forceinline__ bool weighted_shares(long long W, int nw, int cls) {
  return cls > 0 && nw == 3 * cls && W >= static_cast<long long>(kWeightedMinTiles) * nw;
}

// Weight units before work-group i (weighted grid of 3 * cls work-groups).
__device__ __forceinline__ long long slot_weight_before(int cls, int i) {
  if (i < cls) return static_cast<long long>(i) * kSlotWeight0;
  if (i < 2 * cls) return static_cast<long long>(cls) * kSlotWeight0 + static_cast<long long>(i - cls) * kSlotWeight1;
  return static_cast<long long>(cls) * (kSlotWeight0 + kSlotWeight1) +
         static_cast<long long>(i - 2 * cls) * kSlotWeight2;  // (i = 3 * cls: the total)
}

// Work-group i's share starts at tile i*W/nw, or at its weighted place on the weighted grid.
__device__ __forceinline__ long long share_lo(long long W, int nw, int cls, int i) {
  if (!weighted_shares(W, nw, cls)) return (W * i) / nw;
  return (W * slot_weight_before(cls, i)) / (static_cast<long long>(cls) * kSlotWeightSum);
}

// The work-group whose share holds tile t: the largest i with share_lo(i) <= t.
__device__ __forceinline__ int share_owner(long long W, int nw, int cls, long long t) {
  if (!weighted_shares(W, nw, cls)) return static_cast<int>(((t + 1) * nw - 1) / W);
  // share_lo(i) <= t  <=>  slot_weight_before(i) <= X, X = floor(((t + 1) * T - 1) / W)
  const long long T = static_cast<long long>(cls) * kSlotWeightSum;
  const long long X = ((t + 1) * T - 1) / W;
  const long long c1 = static_cast<long long>(cls) * kSlotWeight0;
  const long long c2 = c1 + static_cast<long long>(cls) * kSlotWeight1;
  int i;
  if (X >= c2) i = 2 * cls + static_cast<int>((X - c2) / kSlotWeight2);
  else if (X >= c1) i = cls + static_cast<int>((X - c1) / kSlotWeight1);
  else i = static_cast<int>(X / kSlotWeight0);
  return i < nw - 1 ? i : nw - 1;
}

// Whole work-group: lens_lds[s] = clamped context length of sequence s, pref[s] = blocks of the
// sequences before s, pref[S] = total blocks. Needs blockDim.x a multiple of 64 and at most 1024.
__device__ inline void scan_batch(const DecodeArgs& a, int B, int* lens_lds, int* pref) {
  __shared__ int wave_tot[16];
  const int S = a.num_seqs, nt = blockDim.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nt >> 6;
  const int per = (S + nt - 1) / nt;
  const int beg = tid * per, end = min(S, beg + per);
  const int cap = a.max_blocks * B;
  int local = 0;
  for (int s = beg; s < end; ++s) {
    int L = a.lens[s];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    lens_lds[s] = L;
    local += (L + B - 1) / B;
  }
  int v = local;  // inclusive scan across the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  int excl = before + v - local;
  for (int s = beg; s < end; ++s) {
    pref[s] = excl;
    excl += (lens_lds[s] + B - 1) / B;
  }
  if (tid == nt - 1) {
    int total = 0;
    for (int w = 0; w < nwaves; ++w) total += wave_tot[w];
    pref[S] = total;
  }
  __syncthreads();
}

// Whole work-group: exclusive prefix of `local` over the threads in thread order; *total gets the
// sum. Needs blockDim.x a multiple of 64 and at most 1024.
__device__ inline int block_exclusive_scan(int local, int* total) {
  __shared__ int wave_tot[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  int v = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    before += w < wave ? wave_tot[w] : 0;
    all += wave_tot[w];
  }
  __syncthreads();  // wave_tot may be reused by the next scan
  *total = all;
  return before + v - local;
}

// ---- ordered fixed partitions -------------------------------------------------------------------
//
// With fixed partitions every (sequence, partition) pair is one work-group per unit. Launched in
// partition-major order, the grid ends with the full partitions of the longest sequences: on a
// long-tailed length mix (128 sequences, log-normal median 1024, up to 8192, 1024-token partitions)
// the last of them started some 120 us into a 150 us kernel and ran on an emptying GPU for their
// last 20-30 us, and two thirds of the launched work-groups found an empty partition. The ordered
// grid lists the work longest first: every full partition (sequence-major), then each sequence's
// last, partial partition bucketed by its length, longest bucket first (sequence order within a
// bucket); a sequence with no tokens has one empty item, last, that writes its zero output. Grid
// items past the list end at once. Which work-group computes an item changes nothing in its
// result.

constexpr int kOrderBuckets = 16;
constexpr int kOrderedMaxSeqs = 1024;

// LDS ints the ordering needs for S sequences.
__host__ __device__ constexpr int ordered_lds_ints(int S) { return 2 * S + 1 + kOrderBuckets + 1; }

// Whole work-group (uniform k): the (sequence, partition) of item k of the ordered list, or
// sequence -1 past its end. lds: ordered_lds_ints(S) ints; on return lds[s] is the clamped
// context length of sequence s.
__device__ inline int2 ordered_item(const DecodeArgs& a, int B, long long k, int* lds) {
  const int S = a.num_seqs, nt = blockDim.x, tid = threadIdx.x, pb = a.part_blocks;
  int* lens_l = lds;                // [S]
  int* pref = lds + S;              // [S + 1] full partitions before sequence s
  int* bcnt = pref + S + 1;         // [kOrderBuckets + 1] last partitions per bucket
  __shared__ int found;
  const int per = (S + nt - 1) / nt;
  const int beg = min(S, tid * per), end = min(S, beg + per);
  const int cap = a.max_blocks * B;
  int own_len = 0;  // with one sequence a thread (per == 1): the clamped length of sequence tid
  {
    // The list's length, by every wave on its own (no LDS, no barrier): a work-group past the
    // end leaves here. The grid is sized by the table width, so on long-tailed length mixes most
    // of it lies past the end; the full ordering below would cost each of them 2 us.
    const int lane = tid & 63;
    int items = 0;
    for (int s = lane; s < S; s += 64) {
      int L = a.lens[s];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      if (s == tid) own_len = L;
      const int nblk = (L + B - 1) / B;
      items += nblk == 0 ? 1 : nblk / pb + (nblk % pb != 0 ? 1 : 0);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) items += __shfl_xor(items, off);
    if (k >= items) return make_int2(-1, 0);
  }
  if (tid <= kOrderBuckets) bcnt[tid] = 0;
  __syncthreads();
  // bucket of a sequence's last item: blocks in its partial partition, longest first; a sequence
  // with no tokens goes last; -1: no partial partition
  auto bucket = [&](int nblk) {
    const int rem = nblk % pb;
    return nblk == 0 ? kOrderBuckets - 1 : (rem == 0 ? -1 : (pb - rem) * kOrderBuckets / pb);
  };
  int nfull = 0;
  for (int s = beg; s < end; ++s) {
    int L = own_len;  // (loaded above when per == 1, where s == tid)
    if (per > 1) {
      L = a.lens[s];
      L = L < 0 ? 0 : (L > cap ? cap : L);
    }
    lens_l[s] = L;
    const int nblk = (L + B - 1) / B;
    nfull += nblk / pb;
    const int b = bucket(nblk);
    if (b >= 0) atomicAdd(&bcnt[b], 1);
  }
  int F = 0;
  int excl = block_exclusive_scan(nfull, &F);
  for (int s = beg; s < end; ++s) {
    pref[s] = excl;
    excl += ((lens_l[s] + B - 1) / B) / pb;
  }
  if (tid == 0) pref[S] = F;
  __syncthreads();
  if (k < F) {  // the largest s with pref[s] <= k (its interval [pref[s], pref[s+1]) holds k)
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pref[mid] <= k) lo = mid;
      else hi = mid;
    }
    return make_int2(lo, static_cast<int>(k - pref[lo]));
  }
  long long r = k - F;
  int b = 0;
  for (; b < kOrderBuckets; ++b) {
    if (r < bcnt[b]) break;
    r -= bcnt[b];
  }
  if (b == kOrderBuckets) return make_int2(-1, 0);
  // the r-th sequence (in sequence order) whose last item lies in bucket b
  int mine = 0;
  for (int s = beg; s < end; ++s) mine += bucket((lens_l[s] + B - 1) / B) == b ? 1 : 0;
  int cnt = 0;
  int before = block_exclusive_scan(mine, &cnt);
  if (r >= before && r < before + mine) {
    for (int s = beg; s < end; ++s) {
      if (bucket((lens_l[s] + B - 1) / B) != b) continue;
      if (before == r) found = s;
      ++before;
    }
  }
  __syncthreads();
  const int s = found;
  return make_int2(s, ((lens_l[s] + B - 1) / B) / pb);
}

// ---- the ordered list's items over the XCDs --------------------------------------------------
//
// Work-groups go to the 8 XCDs round-robin by index (work-group w to XCD w mod 8), and each XCD
// dispatches its own in index order. On the MHA decode batch (64 sequences, 40 heads, one item
// per (sequence, head)) the odd-numbered XCDs took 8-13% longer per work-group than the even ones
// for the same items, so with an even split the even XCDs ran out of work 15-20 us before the odd
// ones. The VALU kernel's ordered grid therefore hands the list out in periods of kXcdRounds
// rounds of 8 work-groups, and in the last round of each period the odd-numbered XCDs get an
// empty work-group (it exits at once): they take 8 items for every 9 the even ones take. That
// kernel took 241.4-242.0 us against 246.3-247.0 us for the plain order, its XCDs' mean
// work-group times evened out (59-63 us on every XCD), and the same rounds with the even XCDs
// sitting out took 248.6-249.0 us. Periods of 7 rounds measured the same as 9; 5, 6, 13 and 25
// gained less. (On the GQA batch's MFMA grid the same order measured within 1 us of the plain
// one, so that grid keeps it.) Which work-group takes an item never changes the item's result.

constexpr int kXcdRounds = 9;

// Items one period of kXcdRounds rounds hands out: 8 per round, 4 in the last.
__host__ __device__ constexpr long long xcd_items_per_period() { return 8LL * kXcdRounds - 4; }

// Work-groups of the grid that hands out `items` items (whole periods).
__host__ __device__ constexpr long long xcd_weighted_grid(long long items) {
  return (items + xcd_items_per_period() - 1) / xcd_items_per_period() * 8 * kXcdRounds;
}

// The item of the list work-group w takes, or -1 for an odd-numbered XCD's empty work-group.
__device__ __forceinline__ long long xcd_weighted_item(long long w) {
  const int x = static_cast<int>(w & 7);
  const long long r = w >> 3;
  const int rr = static_cast<int>(r % kXcdRounds);
  const long long per = r / kXcdRounds;
  if (rr == kXcdRounds - 1) {
    if (x & 1) return -1;
    return per * xcd_items_per_period() + 8LL * (kXcdRounds - 1) + (x >> 1);
  }
  return per * xcd_items_per_period() + 8LL * rr + x;
}

// The sequence holding tile t (t < pref[S] * hu): the largest s with pref[s] * hu <= t, which is
// never an empty sequence.
__device__ __forceinline__ int find_seq(const int* pref, int S, long long hu, long long t) {
  int lo = 0, hi = S;  // invariant: pref[lo]*hu <= t < pref[hi]*hu
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<long long>(pref[mid]) * hu <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace pa
