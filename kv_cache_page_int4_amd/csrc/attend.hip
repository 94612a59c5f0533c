// Sparse decode attention over the selected pages (LOCKS abstract: attend only
// the top pages; technical summary sec. 2: every query head of a GQA group
// attends the same page set).
//
// Split-K: the attended page list of a (sequence, KV head) -- the selected
// pages in ascending order, then the partial tail page -- is cut into splits
// of `pages_per_split` pages, one wave each.  The 4 query heads of the group
// share every K/V load.
//  * QK^T on the matrix cores: rows = the 16 tokens of a page, K = head dim,
//    columns = the 4 heads repeated 4 times; lane l gets the logits of tokens
//    4*(l/16) + r (r = 0..3) for head l%4.
//  * softmax in base 2 with an online maximum per 4-page group.
//  * P.V on the vector units: lane l keeps the same 4 tokens and 8 of the
//    128 dims; the 4 heads' probabilities come from its quad by DPP broadcast.
// A second kernel merges the splits by log-sum-exp into bf16 output.
#include "locks_device.h"
#include "locks_internal.h"
#include "select_common.h"

namespace locks {

namespace {

constexpr int kWaves = 4;

struct AttendParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t bs, hs, ts;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* sel;
  const int32_t* sel_count;
  float* part_o;
  float2* part_ml;
  uint16_t* out;
  float* out_lse;
  float scale2;
  int32_t num_blocks, max_pages, budget, hq, hkv, pages_per_split, n_splits;
};

// One wave's split of the attended page list of (sequence b, KV head kvh):
// the first `count` entries of `selrow` (logical pages, ascending; nullptr
// means pages 0..count-1) and then the partial tail page.  `selrow` may point
// to global memory or to LDS.
__device__ __forceinline__ void attend_wave(const AttendParams& p, int split, int kvh, int b,
                                            int count, const int32_t* selrow) {
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, col = lane & 15, h = lane & 3;
  const int qhead0 = kvh * kG;
  {
    int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
    const int n_fin = seq / kB;
    const int tail = seq - n_fin * kB;
    const int n_att = count + (tail > 0 ? 1 : 0);
    const int e0 = split * p.pages_per_split;
    const int e1 = min(e0 + p.pages_per_split, n_att);

    const uint16_t* qrow = p.q + ((size_t)b * p.hq + qhead0 + h) * kD + 32 * row;
    bf16x8 bq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 8 * s));

    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    // page-group bookkeeping: base offset of each page-head and its valid tokens
    auto locate = [&](int eg, size_t off[4], int ntok[4]) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int e = eg + pp;
        int nt = 0, j = -1;
        if (e < e1) {
          if (e < count) {
            j = selrow ? selrow[e] : e;
            nt = (j >= 0 && j < n_fin) ? kB : 0;
          } else {
            j = n_fin;
            nt = tail;
          }
        }
        int bid = (nt > 0) ? bt[j] : 0;
        if ((unsigned)bid >= (unsigned)p.num_blocks) {
          bid = 0;
          nt = 0;
        }
        off[pp] = (size_t)bid * p.bs + (size_t)kvh * p.hs;
        ntok[pp] = nt;
      }
    };
    auto load_k = [&](const size_t off[4], uint4 kr[4][4]) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint16_t* kp = p.kc + off[pp] + (size_t)col * p.ts + 32 * row;
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[pp][s] = *reinterpret_cast<const uint4*>(kp + 8 * s);
      }
    };
    auto load_v = [&](const size_t off[4], uint4 vr[4][4]) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vr[pp][r] = *reinterpret_cast<const uint4*>(p.vc + off[pp] + (size_t)(4 * row + r) * p.ts + 8 * col);
    };

    float M = -INFINITY, lsum = 0.f;
    float acc[4][8];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;

    size_t off[4];
    int ntok[4];
    uint4 kr[4][4], vr[4][4];
    if (e0 < e1) {
      locate(e0, off, ntok);
      load_k(off, kr);
      load_v(off, vr);
    }
    for (int eg = e0; eg < e1; eg += 4) {
      float S[4][4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) a = mfma16x16x32(as_bf16x8(kr[pp][s]), bq[s], a);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[pp][r] = (4 * row + r < ntok[pp]) ? a[r] * p.scale2 : -INFINITY;
      }
      // keys of the next group are fetched while this group finishes
      size_t off_n[4];
      int ntok_n[4];
      const bool more = eg + 4 < e1;
      if (more) {
        locate(eg + 4, off_n, ntok_n);
        load_k(off_n, kr);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[pp][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float Mn = fmaxf(M, mx);
      const float alpha = (Mn == -INFINITY) ? 1.f : fast_exp2(M - Mn);
      float P[4][4];
      float ps = 0.f;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          P[pp][r] = (S[pp][r] == -INFINITY) ? 0.f : fast_exp2(S[pp][r] - Mn);
          ps += P[pp][r];
        }
      lsum = lsum * alpha + ps;
      M = Mn;
      const float al[4] = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha),
                           quad_bcast<3>(alpha)};
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= al[hh];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint4 v = vr[pp][r];
          const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                               bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
          const float p0 = quad_bcast<0>(P[pp][r]), p1 = quad_bcast<1>(P[pp][r]);
          const float p2 = quad_bcast<2>(P[pp][r]), p3 = quad_bcast<3>(P[pp][r]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[0][e] = fmaf(p0, vf[e], acc[0][e]);
            acc[1][e] = fmaf(p1, vf[e], acc[1][e]);
            acc[2][e] = fmaf(p2, vf[e], acc[2][e]);
            acc[3][e] = fmaf(p3, vf[e], acc[3][e]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          off[pp] = off_n[pp];
          ntok[pp] = ntok_n[pp];
        }
        load_v(off, vr);
      }
    }
    // each row of lanes holds a quarter of the tokens: sum the rows
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[hh][e] += __shfl_xor(acc[hh][e], 16);
        acc[hh][e] += __shfl_xor(acc[hh][e], 32);
      }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (row == 0) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        float* o = p.part_o + (((size_t)b * p.hq + qhead0 + hh) * p.n_splits + split) * kD + 8 * col;
        *reinterpret_cast<float4*>(o) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
      }
      if (col < 4)
        p.part_ml[((size_t)b * p.hq + qhead0 + col) * p.n_splits + split] = make_float2(M, lsum);
    }
  }
}

__global__ __launch_bounds__(256) void attend_kernel(AttendParams p) {
  const int split = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int kvh = blockIdx.y, b = blockIdx.z;
  if (split >= p.n_splits) return;
  int count;
  const int32_t* selrow = nullptr;
  if (p.sel) {
    count = max(0, min(p.sel_count[(size_t)b * p.hkv + kvh], p.budget));
    selrow = p.sel + ((size_t)b * p.hkv + kvh) * p.budget;
  } else {
    count = max(0, min(p.seq_lens[b], p.max_pages * kB)) / kB;
  }
  attend_wave(p, split, kvh, b, count, selrow);
}

// ---- final selection fused with the attention --------------------------------
// Every workgroup of a (sequence, KV head) runs the last selection stage
// itself (the top k of that group's chunk candidates, 256 threads), keeps the
// ascending page list in LDS and attends its splits from there: no kernel
// boundary and no global round trip between choosing the pages and reading
// them.  The selection is the same computation as the stand-alone stage, on
// the same candidates in the same order, so its result is identical;
// workgroup 0 also writes it out.
struct FusedSel {
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  int32_t* sel;
  int32_t* sel_count;
  int32_t n_chunks, slots;
};

constexpr int kFusedThreads = 256;

template <int RUN>
__global__ __launch_bounds__(kFusedThreads) void select_attend_kernel(AttendParams p, FusedSel f) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][4];
  __shared__ uint32_t red_smem[3 * (kFusedThreads / 64)];
  __shared__ int scan_smem[kFusedThreads / 64];
  __shared__ int32_t sel_lds[kFusedMaxBudget];

  const int n_cand = f.n_chunks * f.slots;
  const size_t grp = (size_t)b * p.hkv + kvh;
  const uint32_t* gk = f.cand_key + grp * (size_t)n_cand;
  const int32_t* gi = f.cand_idx + grp * (size_t)n_cand;
  const int per = (n_cand + kFusedThreads - 1) / kFusedThreads;
  const int c0 = tid * per;
  uint32_t key[RUN];
  int32_t idx[RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    const int c = c0 + i;
    const bool in = i < per && c < n_cand;
    key[i] = in ? gk[c] : 0u;
    idx[i] = in ? gi[c] : -1;
  }
  int total_valid = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < RUN; ++i)
    if (key[i] != 0u) {
      ++total_valid;
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  sel::block_sum_minmax<kFusedThreads>(total_valid, kmin, kmax, red_smem);
  const int k = min(p.budget, total_valid);
  const bool all = (k >= total_valid);
  uint32_t T = 0u;
  int rem = k;
  if (k > 0 && !all)
    sel::radix_threshold<kFusedThreads>(
        [&](auto fn) {
#pragma unroll
          for (int i = 0; i < RUN; ++i) fn(key[i], key[i] != 0u);
        },
        k, kmin, kmax, hist, sh, &T, &rem);
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    n_gt += (key[i] != 0u && key[i] > T);
    n_eq += (key[i] != 0u && key[i] == T);
  }
  int pos_gt, pos_eq;
  sel::winner_scan<kFusedThreads>(n_gt, n_eq, &pos_gt, &pos_eq, scan_smem);
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (key[i] == 0u || k == 0) continue;
    int at = -1;
    if (key[i] > T) {
      at = pos_gt + min(pos_eq, rem);
      ++pos_gt;
    } else if (key[i] == T) {
      if (pos_eq < rem) at = pos_gt + pos_eq;
      ++pos_eq;
    }
    if (at >= 0 && at < p.budget) sel_lds[at] = idx[i];
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    int32_t* out = f.sel + grp * p.budget;
    for (int s = tid; s < p.budget; s += kFusedThreads) out[s] = (s < k) ? sel_lds[s] : -1;
    if (tid == 0) f.sel_count[grp] = k;
  }
  const int split = blockIdx.x * kWaves + (tid >> 6);
  if (split < p.n_splits) attend_wave(p, split, kvh, b, k, sel_lds);
}

// One workgroup per (sequence, query head): log-sum-exp weights of the
// splits, then out[d] = sum_s w_s o_s[d] / sum_s w_s l_s with independent,
// coalesced loads of the split partials.
constexpr int kMergeW = 4096;

__global__ __launch_bounds__(128) void attend_merge_kernel(AttendParams p) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const size_t row = (size_t)b * p.hq + h;
  const int n = p.n_splits;
  const float2* ml = p.part_ml + row * n;
  __shared__ float wsh[kMergeW];
  __shared__ float red[2];
  float M = -INFINITY;
  for (int s = t; s < n; s += 128) M = fmaxf(M, ml[s].x);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  float L = 0.f;
  for (int s = t; s < n; s += 128) {
    const float2 v = ml[s];
    const float w = (v.x == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(v.x - M);
    if (s < kMergeW) wsh[s] = w;
    L += w * v.y;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = red[0] + red[1];
  const float* po = p.part_o + row * n * kD + t;
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= n; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = po[(size_t)(s + u) * kD];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ss = s + u;
      const float w = (ss < kMergeW) ? wsh[ss]
                    : ((ml[ss].x == -INFINITY) ? 0.f : fast_exp2(ml[ss].x - M));
      acc = fmaf(w, v[u], acc);
    }
  }
  for (; s < n; ++s) {
    const float w = (s < kMergeW) ? wsh[s] : ((ml[s].x == -INFINITY) ? 0.f : fast_exp2(ml[s].x - M));
    acc = fmaf(w, po[(size_t)s * kD], acc);
  }
  p.out[row * kD + t] = (uint16_t)f32_to_bf16((L > 0.f) ? acc / L : 0.f);
  if (p.out_lse && t == 0) p.out_lse[row] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

}  // namespace

bool fused_select_attend_fits(int32_t n_cand, int32_t budget_pages) {
  return budget_pages <= kFusedMaxBudget && n_cand <= 32 * kFusedThreads;
}

hipError_t launch_select_attend(const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, int64_t block_stride,
                                int64_t head_stride, int64_t token_stride, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                                const uint32_t* cand_key, const int32_t* cand_idx,
                                const SelectPlan& sp, int32_t* sel, int32_t* sel_count,
                                int32_t budget_pages, float scale, float* part_o,
                                float2* part_ml, const AttendPlan& plan, uint16_t* out,
                                float* out_lse, hipStream_t stream) {
  AttendParams p{q, k_cache, v_cache, block_stride, head_stride, token_stride, block_table,
                 seq_lens, sel, sel_count, part_o, part_ml, out, out_lse,
                 scale * kLog2e, num_blocks, max_pages, budget_pages, hq, hkv,
                 plan.pages_per_split, plan.n_splits};
  FusedSel f{cand_key, cand_idx, sel, sel_count, sp.n_chunks, sp.slots};
  const int32_t n_cand = sp.n_chunks * sp.slots;
  const int per = (n_cand + kFusedThreads - 1) / kFusedThreads;
  dim3 grid((plan.n_splits + kWaves - 1) / kWaves, hkv, batch);
  if (per <= 4)
    hipLaunchKernelGGL(select_attend_kernel<4>, grid, dim3(kFusedThreads), 0, stream, p, f);
  else if (per <= 16)
    hipLaunchKernelGGL(select_attend_kernel<16>, grid, dim3(kFusedThreads), 0, stream, p, f);
  else
    hipLaunchKernelGGL(select_attend_kernel<32>, grid, dim3(kFusedThreads), 0, stream, p, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(hq, batch), dim3(128), 0, stream, p);
  return hipGetLastError();
}

AttendPlan plan_attend(int32_t batch, int32_t hkv, int32_t max_attended) {
  AttendPlan pl;
  const long long groups = (long long)batch * hkv;
  long long per = 2048 / (groups > 0 ? groups : 1);
  if (per < 1) per = 1;
  long long pages = (max_attended + per - 1) / per;
  pages = ((pages + 3) / 4) * 4;
  if (pages < 4) pages = 4;
  pl.pages_per_split = (int32_t)pages;
  pl.n_splits = (int32_t)((max_attended + pages - 1) / pages);
  if (pl.n_splits < 1) pl.n_splits = 1;
  return pl;
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         int64_t block_stride, int64_t head_stride, int64_t token_stride,
                         int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                         const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                         const int32_t* sel, const int32_t* sel_count, int32_t budget_pages,
                         float scale, float* part_o, float2* part_ml, const AttendPlan& plan,
                         uint16_t* out, float* out_lse, hipStream_t stream) {
  AttendParams p{q, k_cache, v_cache, block_stride, head_stride, token_stride, block_table,
                 seq_lens, sel, sel_count, part_o, part_ml, out, out_lse,
                 scale * kLog2e, num_blocks, max_pages, budget_pages, hq, hkv,
                 plan.pages_per_split, plan.n_splits};
  dim3 grid((plan.n_splits + kWaves - 1) / kWaves, hkv, batch);
  hipLaunchKernelGGL(attend_kernel, grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(hq, batch), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
