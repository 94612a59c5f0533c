// Workgroup-level selection helpers shared by the selection kernels and the
// fused selection + attention kernel: scans, reductions and the radix search
// for the threshold of the k largest 32-bit keys.
#pragma once

#include "locks_device.h"

namespace locks {
namespace sel {

// Exclusive prefix sum over the workgroup of one int per thread; the total
// comes back through `total`.  The cross-wave step is a shuffle scan of the
// wave totals in every wave (no serial loop).  smem >= NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* smem) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = wave_incl_scan(v);
  if (lane == 63) smem[wave] = x;
  __syncthreads();
  const int t = (lane < NW) ? smem[lane] : 0;
  const int u = wave_incl_scan(t);
  // totals of the waves below
  const int before = __builtin_amdgcn_readlane(u, wave) - __builtin_amdgcn_readlane(t, wave);
  *total = __builtin_amdgcn_readlane(u, NW - 1);
  __syncthreads();   // smem is reused by the next call
  return before + x - v;
}

// Workgroup sum of an int and min / max of a uint32 (results in every
// thread).  smem >= 3 * NT/64 words.
template <int NT>
__device__ __forceinline__ void block_sum_minmax(int& sum, uint32_t& mn, uint32_t& mx, uint32_t* smem) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  sum = (int)wave_sum_u((uint32_t)sum);
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  if (lane == 0) {
    smem[wave] = (uint32_t)sum;
    smem[NW + wave] = mn;
    smem[2 * NW + wave] = mx;
  }
  __syncthreads();
  const uint32_t a = (lane < NW) ? smem[lane] : 0u;
  const uint32_t b = (lane < NW) ? smem[NW + lane] : 0xFFFFFFFFu;
  const uint32_t c = (lane < NW) ? smem[2 * NW + lane] : 0u;
  sum = (int)wave_sum_u(a);
  mn = wave_min_u(b);
  mx = wave_max_u(c);
  __syncthreads();
}

// Find the digit bucket holding the rem-th largest key among those counted in
// hist[256] (called by one full wave).  Exactly one lane finds it and stores
// the digit, the rank left inside that bucket and the bucket's population.
__device__ __forceinline__ void pick_digit(const int* hist, int rem, int* sh) {
  const int lane = threadIdx.x & 63;   // lane owns digits 4*lane .. 4*lane+3
  const int4 v = *reinterpret_cast<const int4*>(hist + 4 * lane);
  const int c[4] = {v.x, v.y, v.z, v.w};
  const int tot = c[0] + c[1] + c[2] + c[3];
  const int pre = wave_incl_scan(tot);   // digits up to 4*lane+3
  int above = __builtin_amdgcn_readlane(pre, 63) - pre;  // keys whose digit exceeds 4*lane+3
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    if (above < rem && above + c[e] >= rem) {
      sh[0] = 4 * lane + e;
      sh[1] = rem - above;
      sh[2] = c[e];
    }
    above += c[e];
  }
}

// Threshold T and count `rem` such that the top k keys are exactly the keys
// above T plus the first `rem` keys equal to T (in the callers' order).  The
// radix passes cover only the bits in which the valid keys differ (from their
// min and max), eight at a time from the top, so the first digit already
// spreads the keys over the histogram.  A pass whose boundary bucket is taken
// whole ends the search: T becomes the value just below that bucket and rem
// 0.  A wave whose keys all share one digit adds it with a single atomic.
// Histograms are double-buffered so a pass needs two barriers.
// for_each(f) calls f(key, valid) for each of this thread's slots, the same
// number of times in every thread.  hist: [2][256]; sh: [2][4].
template <int NT, typename ForEach>
__device__ void radix_threshold(ForEach for_each, int k, uint32_t kmin, uint32_t kmax,
                                int (*hist)[256], int (*sh)[4], uint32_t* T_out, int* rem_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0u) {           // every valid key is equal
    *T_out = kmin;
    *rem_out = k;
    return;
  }
  const int hb = 31 - __clz(diff);
  uint32_t pmask = (hb == 31) ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmin & pmask;
  int rem = k;
  for (int i = tid; i < 512; i += NT) hist[i >> 8][i & 255] = 0;
  __syncthreads();
  int buf = 0;
  for (int hi = hb; hi >= 0; hi -= 8) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    for_each([&](uint32_t key, bool valid) {
      const bool in = valid && (key & pmask) == prefix;
      const int dg = in ? (int)((key >> lo) & dmask) : -1;
      const int d0 = __builtin_amdgcn_readfirstlane(dg);
      if (__all(dg == d0)) {
        if (lane == 0 && d0 >= 0) atomicAdd(&hist[buf][d0], 64);
      } else if (in) {
        atomicAdd(&hist[buf][dg], 1);
      }
    });
    __syncthreads();
    if (wave == 0) pick_digit(hist[buf], rem, sh[buf]);
    for (int i = tid; i < 256; i += NT) hist[buf ^ 1][i] = 0;   // next pass's buffer
    __syncthreads();
    prefix |= (uint32_t)sh[buf][0] << lo;
    pmask |= dmask << lo;
    rem = sh[buf][1];
    if (lo > 0 && sh[buf][2] == rem) {
      // the whole boundary bucket is taken: threshold just below it
      *T_out = prefix == 0u ? 0u : prefix - 1u;
      *rem_out = 0;
      return;
    }
    buf ^= 1;
  }
  *T_out = prefix;
  *rem_out = rem;
}

// Ordered compaction of the winners of one workgroup.  A key wins if it is
// above T, or equal to T and among the first `rem` such keys in candidate
// order; both counts come out of one scan of (above << 16 | equal), which is
// exact while a workgroup holds fewer than 2^16 keys.  Returns the numbers of
// above-T and equal-to-T keys before this thread's first one.
template <int NT>
__device__ __forceinline__ void winner_scan(int n_gt, int n_eq, int* pos_gt, int* pos_eq,
                                            int* scan_smem) {
  int tot;
  const int pre = block_exclusive_scan<NT>((n_gt << 16) | n_eq, &tot, scan_smem);
  *pos_gt = pre >> 16;
  *pos_eq = pre & 0xFFFF;
}

}  // namespace sel
}  // namespace locks
