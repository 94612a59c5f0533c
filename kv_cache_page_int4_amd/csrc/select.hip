// Group-shared page selection (LOCKS explainer, technical summary sec. 2:
// group-shared selection; reconstruction and selection).
//
// For a (sequence, selection table) with query heads h of the table -- the
// query heads of one KV head by default, or of several KV heads (one table for
// the whole layer at the widest), the other reading of the group-shared
// table:
//   L_h   = LSE_j s_hat_hj                        (base-2 partials merged)
//   log m_j = log( mean_h exp(s_hat_hj - L_h) )   (kept in the log domain so
//                                                  tiny shares never tie at 0)
// and the k = min(budget, valid pages) largest m_j are kept, ties to the lower
// page index, listed in ascending page order.
//
// Two kernels.  Stage 1: one workgroup per chunk of 2048 pages (4096 when the
// grid would otherwise need a second round) first merges the (max, sum)
// partials of its table's query heads into L_h (one head per wave; a few
// kilobytes per head, cheaper than a kernel boundary), then turns scores into
// order-preserving 32-bit keys and radix-selects the chunk's top
// min(k, chunk pages) (8-bit digits, LDS histograms); survivors are written
// in page order.  Stage 2: one workgroup per (sequence, KV head) radix-selects the
// global top k over all candidates.  Because each chunk emits its survivors in
// page order and chunks are in page order, stream compaction of the winners
// yields ascending page ids directly, and "lowest index among equal keys" is
// "first in candidate order".
#include "locks_device.h"
#include "locks_internal.h"
#include "select_common.h"

namespace locks {

namespace {

using sel::block_exclusive_scan;
using sel::block_sum_minmax;
using sel::radix_threshold;

constexpr int kSelThreads = 1024;   // 16 waves: 4 per SIMD hide the latency chains
// stage-1 workgroups that two per CU run in one round
constexpr long long kSelOneRound = 512;

__global__ __launch_bounds__(kSelThreads) void lse_partials_kernel(
    const float* page_lse, int32_t max_pages, const int32_t* seq_lens, int32_t hq,
    int32_t pending, float2* partials, int32_t n_chunks, int32_t pages_per_chunk) {
  const int chunk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  int seq = max(0, min(seq_lens[b], max_pages * kB));
  const int n_fin = summarized_pages(seq, pending);
  const float* s = page_lse + ((size_t)b * hq + head) * max_pages;
  float m = -INFINITY, sm = 0.f;
  const int j0 = chunk * pages_per_chunk, j1 = min(n_fin, j0 + pages_per_chunk);
  for (int j = j0 + threadIdx.x; j < j1; j += kSelThreads) {
    const float v = s[j] * kLog2e;
    if (v > -INFINITY) lse2_merge(m, sm, v, 1.f);
  }
  wave_lse2(m, sm);
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
  const float2* partials;    // [b][hq][n_partials] base-2 (max, sum) pieces of each head's mass
  int32_t n_partials;
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* sel;
  int32_t* sel_count;
  // ntab: selection tables per sequence; a table holds hq / ntab query heads
  int32_t max_pages, hq, ntab, budget, n_chunks, slots;
  int32_t pending;   // 1: the page holding the newest token is not summarized
};

// Stage 2 over candidates held in registers: thread t owns the contiguous
// run [t*per, t*per + per) of the page-ordered candidate list (per <= RUN), so
// runs are in page order and the ordered compaction is one exclusive scan.
template <int RUN>
__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(SelParams p) {
  const int tab = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][4];
  __shared__ uint32_t red_smem[3 * (kSelThreads / 64)];
  __shared__ int scan_smem[kSelThreads / 64];
  const int n_cand = p.n_chunks * p.slots;
  const size_t grp = (size_t)b * p.ntab + tab;
  const uint32_t* gk = p.cand_key + grp * (size_t)n_cand;
  const int32_t* gi = p.cand_idx + grp * (size_t)n_cand;
  const int per = (n_cand + kSelThreads - 1) / kSelThreads;
  const int c0 = tid * per;
  uint32_t key[RUN];
  int32_t idx[RUN];   // page ids, loaded with the keys (the output needs them last)
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int c = c0 + i;
    const bool in = i < per && c < n_cand;
    key[i] = in ? gk[c] : 0u;
    idx[i] = in ? gi[c] : -1;
  }
  int nv = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (key[i] != 0u) {
      ++nv;
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  int total_valid = nv;
  block_sum_minmax<kSelThreads>(total_valid, kmin, kmax, red_smem);
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
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    n_gt += (key[i] != 0u && key[i] > T);
    n_eq += (key[i] != 0u && key[i] == T);
  }
  int pos_gt, pos_eq;
  sel::winner_scan<kSelThreads>(n_gt, n_eq, &pos_gt, &pos_eq, scan_smem);
  int32_t* out = p.sel + grp * p.budget;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (key[i] == 0u || k == 0) continue;
    bool tk;
    int at;
    if (key[i] > T) {
      tk = true;
      at = pos_gt + min(pos_eq, rem);
      ++pos_gt;
    } else if (key[i] == T) {
      tk = pos_eq < rem;
      at = pos_gt + pos_eq;
      ++pos_eq;
    } else {
      tk = false;
      at = 0;
    }
    if (tk && at < p.budget) out[at] = idx[i];
  }
  for (int s2 = k + tid; s2 < p.budget; s2 += kSelThreads) out[s2] = -1;
  if (tid == 0) p.sel_count[grp] = k;
}

// Stage 2 for candidate lists longer than kSelThreads * 32: the same steps with the
// candidates re-read from memory in every pass (correct, slower).
__global__ __launch_bounds__(kSelThreads) void select_merge_big_kernel(SelParams p) {
  const int tab = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][4];
  __shared__ uint32_t red_smem[3 * (kSelThreads / 64)];
  __shared__ int scan_smem[kSelThreads / 64];
  const int n_cand = p.n_chunks * p.slots;
  const size_t grp = (size_t)b * p.ntab + tab;
  const uint32_t* gk = p.cand_key + grp * (size_t)n_cand;
  const int32_t* gi = p.cand_idx + grp * (size_t)n_cand;
  const int per = (n_cand + kSelThreads - 1) / kSelThreads;
  const int c0 = min(n_cand, tid * per), c1 = min(n_cand, c0 + per);
  auto kread = [&](int c) -> uint32_t { return gk[c]; };
  int nv = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int c = c0; c < c1; ++c) {
    const uint32_t kk = kread(c);
    if (kk != 0u) {
      ++nv;
      kmin = min(kmin, kk);
      kmax = max(kmax, kk);
    }
  }
  int total_valid = nv;
  block_sum_minmax<kSelThreads>(total_valid, kmin, kmax, red_smem);
  const int k = min(p.budget, total_valid);
  const bool all = (k >= total_valid);
  uint32_t T = 0u;
  int rem = k;
  if (k > 0 && !all)
    radix_threshold<kSelThreads>(
        [&](auto f) {
          for (int i = 0; i < per; ++i) {
            const int c = c0 + i;
            const uint32_t kk = (c < c1) ? kread(c) : 0u;
            f(kk, kk != 0u);
          }
        },
        k, kmin, kmax, hist, sh, &T, &rem);
  int n_gt = 0, n_eq = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t kk = kread(c);
    n_gt += (kk != 0u && kk > T);
    n_eq += (kk != 0u && kk == T);
  }
  // candidate lists here may exceed 2^16 entries: two separate scans
  int tot;
  int pos_gt = block_exclusive_scan<kSelThreads>(n_gt, &tot, scan_smem);
  int pos_eq = block_exclusive_scan<kSelThreads>(n_eq, &tot, scan_smem);
  int32_t* out = p.sel + grp * p.budget;
  if (k > 0)
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = kread(c);
      if (kk == 0u) continue;
      if (kk > T) {
        const int at = pos_gt + min(pos_eq, rem);
        if (at < p.budget) out[at] = gi[c];
        ++pos_gt;
      } else if (kk == T) {
        if (pos_eq < rem && pos_gt + pos_eq < p.budget) out[pos_gt + pos_eq] = gi[c];
        ++pos_eq;
      }
    }
  for (int s2 = k + tid; s2 < p.budget; s2 += kSelThreads) out[s2] = -1;
  if (tid == 0) p.sel_count[grp] = k;
}

// PT pages per thread: chunks of kSelThreads * PT pages (2048, or 4096 when the
// grid of 2048-page chunks would not fit the chip in one round).
template <int PT>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8)))
void select_chunk_kernel(SelParams p) {
  constexpr int kPerThread = PT;
  constexpr int kUnroll = (PT == 2) ? 8 : 4;   // partials in flight per lane
  const int chunk = blockIdx.x, tab = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int hpt = p.hq / p.ntab;   // query heads of this table
  int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
  const int n_fin = summarized_pages(seq, p.pending);

  __shared__ int hist[2][256];
  __shared__ int sh[2][4];
  __shared__ uint32_t red_smem[3 * (kSelThreads / 64)];
  __shared__ int scan_smem[kSelThreads / 64];

  // keys of this thread's consecutive pages: log2 sum_h 2^(s_hj log2 e - L_h)
  // over the table's heads.  The heads go in batches of one per wave: each
  // wave first merges its head's (max, sum) partials into L_h (base 2), then
  // every thread adds the batch's heads to its keys, four heads at a time.
  __shared__ float l2s[kSelThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  const int jbase = chunk * (kSelThreads * kPerThread) + kPerThread * tid;
  uint32_t key[kPerThread];
  int nvalid = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    const int jmax = max(n_fin - 1, 0);
    float lm[kPerThread];
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) lm[t] = -INFINITY;
    const int h_end = (tab + 1) * hpt;
    for (int hb = tab * hpt; hb < h_end; hb += kSelThreads / 64) {
      const int nb = min(kSelThreads / 64, h_end - hb);
      __syncthreads();   // the previous batch's normalizers have been read
      if (wave < nb) {
        const float2* pp = p.partials + ((size_t)b * p.hq + hb + wave) * p.n_partials;
        float m = -INFINITY, sm = 0.f;
        for (int c0 = lane; c0 < p.n_partials; c0 += kUnroll * 64) {
          float2 v[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + 64 * u;
            v[u] = (c < p.n_partials) ? pp[c] : make_float2(-INFINITY, 0.f);
          }
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) lse2_merge(m, sm, v[u].x, v[u].y);
        }
        wave_lse2(m, sm);
        if (lane == 0) l2s[wave] = (sm > 0.f) ? m + fast_log2(sm) : -INFINITY;
      }
      __syncthreads();
      // four heads at a time; a head past the batch (tables of 1 or 2 heads)
      // reads a real head's scores but gets the normalizer +inf, so it adds
      // 2^-inf = 0 and leaves the key unchanged
      for (int h0 = hb; h0 < hb + nb; h0 += 4) {
        float sv[4][kPerThread];
        float l2[4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const bool real = h0 + hh < hb + nb;
          const float* s = p.page_lse + ((size_t)b * p.hq + (real ? h0 + hh : h0)) * p.max_pages;
#pragma unroll
          for (int t = 0; t < kPerThread; ++t) sv[hh][t] = s[min(jbase + t, jmax)];
          l2[hh] = real ? l2s[h0 - hb + hh] : INFINITY;
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
#pragma unroll
          for (int t = 0; t < kPerThread; ++t) {
            const float a = sv[hh][t] * kLog2e - l2[hh];
            // log2(2^lm + 2^a) without overflow
            const float hi = fmaxf(lm[t], a), lo = fminf(lm[t], a);
            lm[t] = (hi == -INFINITY) ? -INFINITY : hi + fast_log2(1.f + fast_exp2(lo - hi));
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
      const bool ok = (jbase + t < n_fin) && (lm[t] > -INFINITY) && (lm[t] < INFINITY);
      key[t] = ok ? float_key(lm[t]) : 0u;   // 0 = absent (no finite float maps to 0)
      nvalid += ok;
      if (ok) {
        kmin = min(kmin, key[t]);
        kmax = max(kmax, key[t]);
      }
    }
  }
  int total_valid = nvalid;
  block_sum_minmax<kSelThreads>(total_valid, kmin, kmax, red_smem);
  const int kc = min(p.budget, total_valid);

  // radix select of the kc-th largest key
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
  // winners: key > T, or key == T among the first `rem` in page order (T = 0
  // when every valid key is kept)
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t) {
    n_gt += (key[t] != 0u && key[t] > T);
    n_eq += (key[t] != 0u && key[t] == T);
  }
  int pos_gt, pos_eq;
  sel::winner_scan<kSelThreads>(n_gt, n_eq, &pos_gt, &pos_eq, scan_smem);
  const size_t grp = (size_t)b * p.ntab + tab;
  const size_t cbase = (grp * (size_t)p.n_chunks + chunk) * p.slots;
#pragma unroll
  for (int t = 0; t < kPerThread; ++t) {
    if (key[t] == 0u || kc == 0) continue;
    int at = -1;
    if (key[t] > T) {
      at = pos_gt + min(pos_eq, rem);
      ++pos_gt;
    } else if (key[t] == T) {
      if (pos_eq < rem) at = pos_gt + pos_eq;
      ++pos_eq;
    }
    if (at >= 0) {
      p.cand_key[cbase + at] = key[t];
      p.cand_idx[cbase + at] = jbase + t;
    }
  }
  for (int s = kc + tid; s < p.slots; s += kSelThreads) {
    p.cand_key[cbase + s] = 0u;
    p.cand_idx[cbase + s] = -1;
  }
}

}  // namespace

SelectPlan plan_select(int32_t max_pages, int32_t budget_pages, int64_t groups) {
  SelectPlan pl;
  pl.chunk_pages = kSelChunk;
  if ((long long)((max_pages + kSelChunk - 1) / kSelChunk) * groups > kSelOneRound)
    pl.chunk_pages = 2 * kSelChunk;
  pl.n_chunks = (max_pages + pl.chunk_pages - 1) / pl.chunk_pages;
  pl.slots = budget_pages < pl.chunk_pages ? budget_pages : pl.chunk_pages;
  if (pl.slots < 1) pl.slots = 1;
  return pl;
}

hipError_t launch_lse_partials(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                               int32_t batch, int32_t hq, int32_t pending, float2* partials,
                               int32_t n_chunks, int32_t pages_per_chunk, hipStream_t stream) {
  hipLaunchKernelGGL(lse_partials_kernel, dim3(n_chunks, hq, batch), dim3(kSelThreads), 0, stream,
                     page_lse, max_pages, seq_lens, hq, pending, partials, n_chunks,
                     pages_per_chunk);
  return hipGetLastError();
}

hipError_t launch_select_stage1(const float* page_lse, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t ntab,
                                int32_t pending, int32_t budget_pages, const float2* partials,
                                int32_t n_partials, uint32_t* cand_key,
                                int32_t* cand_idx, const SelectPlan& plan, hipStream_t stream) {
  SelParams p{page_lse, seq_lens, partials, n_partials, cand_key, cand_idx, nullptr, nullptr,
              max_pages, hq, ntab, budget_pages, plan.n_chunks, plan.slots, pending};
  const dim3 grid(plan.n_chunks, ntab, batch);
  if (plan.chunk_pages > kSelChunk)
    hipLaunchKernelGGL(select_chunk_kernel<2 * kSelChunk / kSelThreads>, grid, dim3(kSelThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL(select_chunk_kernel<kSelChunk / kSelThreads>, grid, dim3(kSelThreads), 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_select(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                         int32_t batch, int32_t hq, int32_t ntab, int32_t pending,
                         int32_t budget_pages, const float2* partials, int32_t n_partials,
                         uint32_t* cand_key, int32_t* cand_idx, const SelectPlan& plan,
                         int32_t* sel, int32_t* sel_count, hipStream_t stream) {
  hipError_t e = launch_select_stage1(page_lse, max_pages, seq_lens, batch, hq, ntab, pending,
                                      budget_pages, partials, n_partials, cand_key, cand_idx,
                                      plan, stream);
  if (e != hipSuccess) return e;
  SelParams p{page_lse, seq_lens, partials, n_partials, cand_key, cand_idx, sel, sel_count,
              max_pages, hq, ntab, budget_pages, plan.n_chunks, plan.slots, pending};
  const int per = (plan.n_chunks * plan.slots + kSelThreads - 1) / kSelThreads;
  if (per <= 8)
    hipLaunchKernelGGL(select_merge_kernel<8>, dim3(ntab, batch), dim3(kSelThreads), 0, stream, p);
  else if (per <= 32)
    hipLaunchKernelGGL(select_merge_kernel<32>, dim3(ntab, batch), dim3(kSelThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(select_merge_big_kernel, dim3(ntab, batch), dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
