// Group-shared page selection (LOCKS explainer, technical summary sec. 2:
// group-shared selection; reconstruction and selection).
//
// For a (sequence, KV head) with query heads h of the group:
//   L_h   = LSE_j s_hat_hj                        (base-2 partials merged)
//   log m_j = log( mean_h exp(s_hat_hj - L_h) )   (kept in the log domain so
//                                                  tiny shares never tie at 0)
// and the k = min(budget, valid pages) largest m_j are kept, ties to the lower
// page index, listed in ascending page order.
//
// Two kernels.  Stage 1: one workgroup per 2048-page chunk turns scores into
// order-preserving 32-bit keys and radix-selects the chunk's top min(k, 2048)
// (8-bit digits, LDS histograms); survivors are written in page order.
// Stage 2: one workgroup per (sequence, KV head) radix-selects the global top
// k over all candidates, staged in LDS when they fit.  Because each chunk emits its survivors
// in page order and chunks are in page order, stream compaction of the
// winners yields ascending page ids directly, and "lowest index among equal
// keys" is "first in candidate order".
#include "locks_device.h"
#include "locks_internal.h"

namespace locks {

namespace {

constexpr int kSelThreads = 1024;   // 16 waves: 4 per SIMD hide the latency chains
constexpr int kPerThread = kSelChunk / kSelThreads;  // 2

// Inclusive prefix sum over a workgroup (blockDim.x <= 1024), returns the
// exclusive prefix and the total through `total`.
template <int NT>
__device__ int block_exclusive_scan(int v, int* total, int* smem /* >= NT/64 + 1 */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) smem[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int t = smem[w];
      smem[w] = run;
      run += t;
    }
    smem[NT / 64] = run;
  }
  __syncthreads();
  const int excl = smem[wave] + x - v;
  *total = smem[NT / 64];
  __syncthreads();
  return excl;
}

// Block-wide min and max (result in every thread); smem >= NT/64 + 1 ints.
template <int NT>
__device__ void block_minmax(uint32_t& mn, uint32_t& mx, int* smem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  __shared__ uint32_t red[2][NT / 64];
  if (lane == 0) {
    red[0][wave] = mn;
    red[1][wave] = mx;
  }
  __syncthreads();
  mn = red[0][0];
  mx = red[1][0];
  for (int w = 1; w < NT / 64; ++w) {
    mn = min(mn, red[0][w]);
    mx = max(mx, red[1][w]);
  }
  __syncthreads();
  (void)smem;
}

// Find the digit bucket holding the rem-th largest key among those counted in
// hist[256] (called by one full wave).  Exactly one lane finds it and stores
// the digit and the rank left inside that bucket.
__device__ void pick_digit(const int* hist, int rem, int* sh_digit, int* sh_rem) {
  const int lane = threadIdx.x & 63;   // lane owns digits 4*lane .. 4*lane+3
  int c[4], tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = hist[4 * lane + e];
    tot += c[e];
  }
  int x = tot;  // inclusive suffix sum over lanes (higher digits first)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(x, o);
    if (lane + o < 64) x += y;
  }
  int above = x - tot;  // keys whose digit exceeds 4*lane+3
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    if (above < rem && above + c[e] >= rem) {
      *sh_digit = 4 * lane + e;
      *sh_rem = rem - above;
    }
    above += c[e];
  }
}

// Threshold T of the k-th largest key and the number `rem` of keys equal to T
// that belong to the top k.  The radix passes cover only the bits in which
// the keys differ (from the block-wide min and max of the valid keys), eight
// at a time from the top, so the first digit already spreads the keys over
// the histogram; a wave whose keys all share one digit adds it with a single
// atomic.  Histograms are double-buffered so a pass needs two barriers.
// for_each(f) calls f(key, valid) for each of this thread's slots, the same
// number of times in every thread.  hist: [2][256]; sh: [2][2].
template <int NT, typename ForEach>
__device__ void radix_threshold(ForEach for_each, int k, uint32_t kmin, uint32_t kmax,
                                int (*hist)[256], int (*sh)[2], uint32_t* T_out, int* rem_out) {
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
    if (wave == 0) pick_digit(hist[buf], rem, &sh[buf][0], &sh[buf][1]);
    for (int i = tid; i < 256; i += NT) hist[buf ^ 1][i] = 0;   // next pass's buffer
    __syncthreads();
    prefix |= (uint32_t)sh[buf][0] << lo;
    pmask |= dmask << lo;
    rem = sh[buf][1];
    buf ^= 1;
  }
  *T_out = prefix;
  *rem_out = rem;
}

__global__ __launch_bounds__(kSelThreads) void lse_partials_kernel(
    const float* page_lse, int32_t max_pages, const int32_t* seq_lens, int32_t hq,
    float2* partials, int32_t n_chunks, int32_t pages_per_chunk) {
  const int chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  int seq = max(0, min(seq_lens[b], max_pages * kB));
  const int n_fin = seq / kB;
  const float* s = page_lse + ((size_t)b * hq + head) * max_pages;
  float m = -INFINITY, sm = 0.f;
  const int j0 = chunk * pages_per_chunk, j1 = min(n_fin, j0 + pages_per_chunk);
  for (int j = j0 + threadIdx.x; j < j1; j += kSelThreads) {
    const float v = s[j] * kLog2e;
    if (v > -INFINITY) lse2_merge(m, sm, v, 1.f);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sm, o);
    lse2_merge(m, sm, m2, s2);
  }
  __shared__ float2 red[kSelThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(m, sm);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kSelThreads / 64; ++w) lse2_merge(m, sm, red[w].x, red[w].y);
    partials[((size_t)b * hq + head) * n_chunks + chunk] = make_float2(m, sm);
  }
}

struct SelParams {
  const float* page_lse;
  const int32_t* seq_lens;
  const float2* partials;
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* sel;
  int32_t* sel_count;
  int32_t max_pages, hq, hkv, budget, n_partials, n_chunks, slots;
};

// Stage 2 over candidates held in registers: thread t owns the contiguous
// run [t*per, t*per + per) of the page-ordered candidate list (per <= RUN), so
// runs are in page order and the ordered compaction is one exclusive scan.
template <int RUN>
__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(SelParams p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][2];
  __shared__ int scan_smem[kSelThreads / 64 + 1];
  const int n_cand = p.n_chunks * p.slots;
  const size_t gbase = ((size_t)b * p.hkv + kvh) * (size_t)n_cand;
  const uint32_t* gk = p.cand_key + gbase;
  const int32_t* gi = p.cand_idx + gbase;
  const int per = (n_cand + kSelThreads - 1) / kSelThreads;
  const int c0 = tid * per;
  uint32_t key[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int c = c0 + i;
    key[i] = (i < per && c < n_cand) ? gk[c] : 0u;
  }
  int nv = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < RUN; ++i)
    if (key[i] != 0u) {
      ++nv;
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  int total_valid;
  (void)block_exclusive_scan<kSelThreads>(nv, &total_valid, scan_smem);
  block_minmax<kSelThreads>(kmin, kmax, scan_smem);
  const int k = min(p.budget, total_valid);
  const bool all = (k >= total_valid);
  uint32_t T = 0u;
  int rem = k;
  if (k > 0 && !all)
    radix_threshold<kSelThreads>(
        [&](auto f) {
#pragma unroll
          for (int i = 0; i < RUN; ++i) f(key[i], key[i] != 0u);
        },
        k, kmin, kmax, hist, sh, &T, &rem);
  int neq = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) neq += (!all && key[i] != 0u && key[i] == T);
  int tot_eq;
  const int eq_before = block_exclusive_scan<kSelThreads>(neq, &tot_eq, scan_smem);
  uint32_t take = 0u;   // bit i: slot i is a winner
  int ntake = 0;
  {
    int eqr = eq_before;
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      bool tk = false;
      if (key[i] != 0u && k > 0) {
        if (all || key[i] > T) tk = true;
        else if (key[i] == T) tk = (eqr++ < rem);
      }
      take |= (tk ? 1u : 0u) << i;
      ntake += tk;
    }
  }
  int tot_take;
  int pos = block_exclusive_scan<kSelThreads>(ntake, &tot_take, scan_smem);
  int32_t* out = p.sel + ((size_t)b * p.hkv + kvh) * p.budget;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if ((take >> i) & 1u) {
      if (pos < p.budget) out[pos] = gi[c0 + i];
      ++pos;
    }
  }
  const int written = min(tot_take, p.budget);
  for (int s2 = written + tid; s2 < p.budget; s2 += kSelThreads) out[s2] = -1;
  if (tid == 0) p.sel_count[(size_t)b * p.hkv + kvh] = written;
}

// Stage 2 for candidate lists longer than kSelThreads * 32: the same steps with the
// candidates re-read from memory in every pass (correct, slower).
__global__ __launch_bounds__(kSelThreads) void select_merge_big_kernel(SelParams p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][2];
  __shared__ int scan_smem[kSelThreads / 64 + 1];
  const int n_cand = p.n_chunks * p.slots;
  const size_t gbase = ((size_t)b * p.hkv + kvh) * (size_t)n_cand;
  const uint32_t* gk = p.cand_key + gbase;
  const int32_t* gi = p.cand_idx + gbase;
  const int per = (n_cand + kSelThreads - 1) / kSelThreads;
  const int c0 = min(n_cand, tid * per), c1 = min(n_cand, c0 + per);
  int nv = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int c = c0; c < c1; ++c) {
    const uint32_t kk = gk[c];
    if (kk != 0u) {
      ++nv;
      kmin = min(kmin, kk);
      kmax = max(kmax, kk);
    }
  }
  int total_valid;
  (void)block_exclusive_scan<kSelThreads>(nv, &total_valid, scan_smem);
  block_minmax<kSelThreads>(kmin, kmax, scan_smem);
  const int k = min(p.budget, total_valid);
  const bool all = (k >= total_valid);
  uint32_t T = 0u;
  int rem = k;
  if (k > 0 && !all)
    radix_threshold<kSelThreads>(
        [&](auto f) {
          for (int i = 0; i < per; ++i) {
            const int c = c0 + i;
            const uint32_t kk = (c < c1) ? gk[c] : 0u;
            f(kk, kk != 0u);
          }
        },
        k, kmin, kmax, hist, sh, &T, &rem);
  int neq = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t kk = gk[c];
    neq += (!all && kk != 0u && kk == T);
  }
  int tot_eq;
  const int eq_before = block_exclusive_scan<kSelThreads>(neq, &tot_eq, scan_smem);
  auto winner = [&](uint32_t kk, int& eqr) -> bool {
    if (kk == 0u || k == 0) return false;
    if (all || kk > T) return true;
    if (kk == T) return eqr++ < rem;
    return false;
  };
  int ntake = 0;
  {
    int eqr = eq_before;
    for (int c = c0; c < c1; ++c) ntake += winner(gk[c], eqr);
  }
  int tot_take;
  int pos = block_exclusive_scan<kSelThreads>(ntake, &tot_take, scan_smem);
  int32_t* out = p.sel + ((size_t)b * p.hkv + kvh) * p.budget;
  {
    int eqr = eq_before;
    for (int c = c0; c < c1; ++c)
      if (winner(gk[c], eqr)) {
        if (pos < p.budget) out[pos] = gi[c];
        ++pos;
      }
  }
  const int written = min(tot_take, p.budget);
  for (int s2 = written + tid; s2 < p.budget; s2 += kSelThreads) out[s2] = -1;
  if (tid == 0) p.sel_count[(size_t)b * p.hkv + kvh] = written;
}

__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(SelParams p) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
  const int n_fin = seq / kB;

  __shared__ float L2[kG];
  __shared__ float2 wpart[kSelThreads / 64];
  __shared__ int hist[2][256];
  __shared__ int sh[2][2];
  __shared__ int scan_smem[kSelThreads / 64 + 1];

  // scores of this thread's pages: 4 x kPerThread loads (clamped in-bounds
  // index), issued before the normalizer so that both are in flight together
  const int jbase = chunk * kSelChunk + kPerThread * tid;
  float sv[kG][kPerThread];
  {
    const int jmax = max(n_fin - 1, 0);
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      const float* s = p.page_lse + ((size_t)b * p.hq + kvh * kG + hh) * p.max_pages;
#pragma unroll
      for (int t = 0; t < kPerThread; ++t) sv[hh][t] = s[min(jbase + t, jmax)];
    }
  }

  // per-head normalizer from the scoring partials: waves 4h..4h+3 merge head
  // h's partials, 16 independent loads per lane per round
  {
    constexpr int kWavesPerHead = kSelThreads / 64 / kG;
    constexpr int kU = 16;
    const int hh = wave / kWavesPerHead, part = wave % kWavesPerHead;
    const float2* pp = p.partials + ((size_t)b * p.hq + kvh * kG + hh) * p.n_partials;
    float m = -INFINITY, s = 0.f;
    for (int c0 = part * 64 + lane; c0 < p.n_partials; c0 += kU * kWavesPerHead * 64) {
      float2 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + kWavesPerHead * 64 * u;
        v[u] = (c < p.n_partials) ? pp[c] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) lse2_merge(m, s, v[u].x, v[u].y);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
      lse2_merge(m, s, m2, s2);
    }
    if (lane == 0) wpart[wave] = make_float2(m, s);
    __syncthreads();
    if (tid < kG) {
      float mm = -INFINITY, ss = 0.f;
#pragma unroll
      for (int i = 0; i < kWavesPerHead; ++i) {
        const float2 v = wpart[tid * kWavesPerHead + i];
        lse2_merge(mm, ss, v.x, v.y);
      }
      L2[tid] = (ss > 0.f) ? mm + fast_log2(ss) : -INFINITY;
    }
    __syncthreads();
  }

  // keys of this thread's consecutive pages
  uint32_t key[kPerThread];
  int nvalid = 0;
  {
    float lm[kPerThread];
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) lm[t] = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      const float l2 = L2[hh];
#pragma unroll
      for (int t = 0; t < kPerThread; ++t) {
        const float a = sv[hh][t] * kLog2e - l2;
        // log2(2^lm + 2^a) without overflow
        const float hi = fmaxf(lm[t], a), lo = fminf(lm[t], a);
        lm[t] = (hi == -INFINITY) ? -INFINITY : hi + fast_log2(1.f + fast_exp2(lo - hi));
      }
    }
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
      const bool ok = (jbase + t < n_fin) && (lm[t] > -INFINITY) && (lm[t] < INFINITY);
      key[t] = ok ? float_key(lm[t]) : 0u;   // 0 = absent (no finite float maps to 0)
      nvalid += ok;
    }
  }
  int total_valid;
  (void)block_exclusive_scan<kSelThreads>(nvalid, &total_valid, scan_smem);
  const int kc = min(p.budget, total_valid);

  // radix select of the kc-th largest key
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t)
    if (key[t] != 0u) {
      kmin = min(kmin, key[t]);
      kmax = max(kmax, key[t]);
    }
  block_minmax<kSelThreads>(kmin, kmax, scan_smem);
  uint32_t T = 0u;
  int rem = kc;
  if (kc > 0 && kc < total_valid) {
    radix_threshold<kSelThreads>(
        [&](auto f) {
#pragma unroll
          for (int t = 0; t < kPerThread; ++t) f(key[t], key[t] != 0u);
        },
        kc, kmin, kmax, hist, sh, &T, &rem);
  }
  // winners: key > T, or key == T among the first `rem` in page order
  const bool all = (kc >= total_valid);
  int neq = 0;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t) neq += (!all && key[t] != 0u && key[t] == T);
  int tot_eq;
  int eq_before = block_exclusive_scan<kSelThreads>(neq, &tot_eq, scan_smem);
  bool take[kPerThread];
  int ntake = 0;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t) {
    bool tk;
    if (key[t] == 0u) tk = false;
    else if (all || kc == 0) tk = all;
    else if (key[t] > T) tk = true;
    else if (key[t] == T) tk = (eq_before++ < rem);
    else tk = false;
    take[t] = tk;
    ntake += tk;
  }
  int tot_take;
  int pos = block_exclusive_scan<kSelThreads>(ntake, &tot_take, scan_smem);
  const size_t gbase = ((size_t)b * p.hkv + kvh) * (size_t)p.n_chunks * p.slots;
  const size_t cbase = gbase + (size_t)chunk * p.slots;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t) {
    if (take[t]) {
      p.cand_key[cbase + pos] = key[t];
      p.cand_idx[cbase + pos] = jbase + t;
      ++pos;
    }
  }
  for (int s = tot_take + tid; s < p.slots; s += kSelThreads) {
    p.cand_key[cbase + s] = 0u;
    p.cand_idx[cbase + s] = -1;
  }

}

}  // namespace

SelectPlan plan_select(int32_t max_pages, int32_t budget_pages) {
  SelectPlan pl;
  pl.n_chunks = (max_pages + kSelChunk - 1) / kSelChunk;
  pl.slots = budget_pages < kSelChunk ? budget_pages : kSelChunk;
  if (pl.slots < 1) pl.slots = 1;
  return pl;
}

hipError_t launch_lse_partials(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                               int32_t batch, int32_t hq, float2* partials, int32_t n_chunks,
                               int32_t pages_per_chunk, hipStream_t stream) {
  hipLaunchKernelGGL(lse_partials_kernel, dim3(n_chunks, hq, batch), dim3(kSelThreads), 0, stream,
                     page_lse, max_pages, seq_lens, hq, partials, n_chunks, pages_per_chunk);
  return hipGetLastError();
}

hipError_t launch_select(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                         int32_t batch, int32_t hq, int32_t hkv, int32_t budget_pages,
                         const float2* partials, int32_t n_partials, uint32_t* cand_key,
                         int32_t* cand_idx, const SelectPlan& plan, int32_t* sel,
                         int32_t* sel_count, hipStream_t stream) {
  SelParams p{page_lse, seq_lens, partials, cand_key, cand_idx, sel, sel_count,
              max_pages, hq, hkv, budget_pages, n_partials, plan.n_chunks, plan.slots};
  hipLaunchKernelGGL(select_chunk_kernel, dim3(plan.n_chunks, hkv, batch), dim3(kSelThreads), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = (plan.n_chunks * plan.slots + kSelThreads - 1) / kSelThreads;
  if (per <= 8)
    hipLaunchKernelGGL(select_merge_kernel<8>, dim3(hkv, batch), dim3(kSelThreads), 0, stream, p);
  else if (per <= 32)
    hipLaunchKernelGGL(select_merge_kernel<32>, dim3(hkv, batch), dim3(kSelThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(select_merge_big_kernel, dim3(hkv, batch), dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
