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
// Two stages.  Stage 1: one workgroup per 2048-page chunk turns scores into
// order-preserving 32-bit keys in LDS and radix-selects the chunk's top
// min(k, 2048) (8-bit digits, LDS histograms); survivors are written in page
// order.  Stage 2: one workgroup per (sequence, KV head) radix-selects the
// global top k over the candidates.  Because each chunk emits its survivors
// in page order and chunks are in page order, stream compaction of the
// winners yields ascending page ids directly, and "lowest index among equal
// keys" is "first in candidate order".
#include "locks_device.h"
#include "locks_internal.h"

namespace locks {

namespace {

constexpr int kSelThreads = 256;
constexpr int kPerThread = kSelChunk / kSelThreads;  // 8
constexpr int kMergeThreads = 1024;

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

__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(SelParams p) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
  const int n_fin = seq / kB;

  __shared__ float L2[kG];
  __shared__ int hist[256];
  __shared__ int scan_smem[kSelThreads / 64 + 1];
  __shared__ int sh_digit, sh_rem;

  // per-head normalizer from the scoring partials (wave w -> head w)
  {
    const float2* pp = p.partials + ((size_t)b * p.hq + kvh * kG + wave) * p.n_partials;
    float m = -INFINITY, s = 0.f;
    for (int c = lane; c < p.n_partials; c += 64) lse2_merge(m, s, pp[c].x, pp[c].y);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
      lse2_merge(m, s, m2, s2);
    }
    if (lane == 0) L2[wave] = (s > 0.f) ? m + fast_log2(s) : -INFINITY;
  }
  __syncthreads();

  // keys of this thread's 8 consecutive pages
  const int jbase = chunk * kSelChunk + kPerThread * tid;
  uint32_t key[kPerThread];
  int nvalid = 0;
  {
    float lm[kPerThread];
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) lm[t] = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      const float* s = p.page_lse + ((size_t)b * p.hq + kvh * kG + hh) * p.max_pages;
      const float l2 = L2[hh];
#pragma unroll
      for (int t = 0; t < kPerThread; ++t) {
        const int j = jbase + t;
        if (j < n_fin) {
          const float a = s[j] * kLog2e - l2;
          // log2(2^lm + 2^a) without overflow
          const float hi = fmaxf(lm[t], a), lo = fminf(lm[t], a);
          lm[t] = (hi == -INFINITY) ? -INFINITY : hi + fast_log2(1.f + fast_exp2(lo - hi));
        }
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
  uint32_t prefix = 0, pmask = 0;
  int rem = kc;
  if (kc > 0 && kc < total_valid) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kPerThread; ++t)
        if (key[t] != 0u && (key[t] & pmask) == prefix) atomicAdd(&hist[(key[t] >> shift) & 255], 1);
      __syncthreads();
      if (wave == 0) pick_digit(hist, rem, &sh_digit, &sh_rem);
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= 0xFFu << shift;
      rem = sh_rem;
      __syncthreads();
    }
  }
  // winners: key > T, or key == T among the first `rem` in page order
  const uint32_t T = prefix;
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
  const size_t cbase = (((size_t)b * p.hkv + kvh) * p.n_chunks + chunk) * p.slots;
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

__global__ __launch_bounds__(kMergeThreads) void select_merge_kernel(SelParams p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_cand = p.n_chunks * p.slots;
  const size_t cbase = ((size_t)b * p.hkv + kvh) * (size_t)n_cand;
  const uint32_t* ck = p.cand_key + cbase;
  const int32_t* ci = p.cand_idx + cbase;

  __shared__ int hist[256];
  __shared__ int scan_smem[kMergeThreads / 64 + 1];
  __shared__ int sh_digit, sh_rem;

  int nv = 0;
  for (int c = tid; c < n_cand; c += kMergeThreads) nv += (ck[c] != 0u);
  int total_valid;
  (void)block_exclusive_scan<kMergeThreads>(nv, &total_valid, scan_smem);
  const int k = min(p.budget, total_valid);

  uint32_t prefix = 0, pmask = 0;
  int rem = k;
  const bool all = (k >= total_valid);
  if (k > 0 && !all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int c = tid; c < n_cand; c += kMergeThreads) {
        const uint32_t kk = ck[c];
        if (kk != 0u && (kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) pick_digit(hist, rem, &sh_digit, &sh_rem);
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= 0xFFu << shift;
      rem = sh_rem;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;
  int32_t* out = p.sel + ((size_t)b * p.hkv + kvh) * p.budget;
  // ordered compaction, one tile of kMergeThreads candidates at a time
  int written = 0, eq_seen = 0;
  for (int base = 0; base < n_cand; base += kMergeThreads) {
    const int c = base + tid;
    const uint32_t kk = (c < n_cand) ? ck[c] : 0u;
    const bool is_eq = (!all && kk != 0u && kk == T);
    int tot_eq;
    const int eq_rank = eq_seen + block_exclusive_scan<kMergeThreads>(is_eq ? 1 : 0, &tot_eq, scan_smem);
    bool tk = false;
    if (kk != 0u) {
      if (all) tk = true;
      else if (kk > T) tk = true;
      else if (is_eq) tk = eq_rank < rem;
    }
    if (k == 0) tk = false;
    int tot_take;
    const int pos = written + block_exclusive_scan<kMergeThreads>(tk ? 1 : 0, &tot_take, scan_smem);
    if (tk && pos < p.budget) out[pos] = ci[c];
    written += tot_take;
    eq_seen += tot_eq;
  }
  for (int s = min(written, p.budget) + tid; s < p.budget; s += kMergeThreads) out[s] = -1;
  if (tid == 0) p.sel_count[(size_t)b * p.hkv + kvh] = min(written, p.budget);
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
  hipLaunchKernelGGL(select_merge_kernel, dim3(hkv, batch), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
