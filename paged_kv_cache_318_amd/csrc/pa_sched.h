// Balanced work split for the decode kernels (device side).
//
// The batch's work is the flattened list of (sequence, unit, block) tiles, sequence-major: a
// "unit" is what one work-group accumulates (a query head for the VALU kernel, a kv head with its
// query group for the MFMA kernel), and unit (s, x) owns nblk(s) consecutive tiles. With W tiles
// in all and nw work-groups, work-group i takes tiles [i*W/nw, (i+1)*W/nw): every work-group gets
// the same amount of K/V to read whatever the length mix, so there is no tail of long work-groups.
// A unit cut by a share boundary is finished by the merge kernel from the partial results of the
// work-groups that share it (at most two partial results per work-group: its first and its last
// unit), combined with the same log-sum-exp algebra as the rest of the method.
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

// Work-group i's share starts at tile i*W/nw.
__device__ __forceinline__ long long share_lo(long long W, int nw, int i) {
  return (W * i) / nw;
}

// The work-group whose share holds tile t: the largest i with share_lo(i) <= t.
__device__ __forceinline__ int share_owner(long long W, int nw, long long t) {
  return static_cast<int>(((t + 1) * nw - 1) / W);
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
