// Exact page log-sum-exp from the true keys: s_hj = LSE_i(q_h . k_ij / sqrt(d))
// over the 16 tokens of every summarized page.  This is the "read every key"
// selector the LOCKS pages compare against (LOCKS explainer, technical summary
// sec. 3, contributions: selection quality against exact page attention mass).
// Its output has the layout of the estimated page LSE, so the same selection
// kernels turn it into the exact top-k page set.
//
// Work split: one-wave workgroups, W per (sequence, KV head); workgroup w
// takes the kExactPages consecutive pages from w * kExactPages on, and writes
// each head's run of page LSEs at the end as whole 64-byte pieces.  A
// page-head (16 x 128 bf16 = 4 KB) is read by the 64 lanes as 64 contiguous
// bytes each (token lane%16, dims 32*(lane/16)..+32), two pages ahead of the
// one being computed.
//  * QK^T on the matrix cores: rows = the 16 tokens, K = head dim, columns =
//    4 query heads repeated 4 times; lane l gets tokens 4*(l/16)+r
//    (r = 0..3) of head slot l%4.  A GQA group of 8 heads takes two such
//    4-head sub-passes over the same keys; a group of 1 or 2 fills the 4
//    slots with its heads repeated.
//  * LSE over the 16 tokens: max and sum over the 4 registers, then over the
//    lanes 16 and 32 apart.
#include "locks_device.h"
#include "locks_internal.h"

#include <algorithm>

namespace locks {

namespace {

constexpr int kExactPages = 16;   // pages per workgroup

struct ExactParams {
  const uint16_t* q;
  const uint16_t* kc;
  int64_t bs, hs, ts;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* page_lse;
  float scale2;   // softmax scale * log2(e)
  int32_t num_blocks, max_pages, hq, hkv, n_wg;
  int32_t group;   // query heads per KV head (1, 2, 4 or 8)
  int32_t pending; // 1: the page holding the newest token is not summarized
};

// NSUB: 4-head sub-passes (2 for a group of 8 heads, else 1).
template <int NSUB>
__global__ __launch_bounds__(64) void exact_lse_kernel(ExactParams p) {
  constexpr int kSlots = 4 * NSUB;
  const int lane = threadIdx.x;
  const int w = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int W = p.n_wg;
  const int G = p.group;
  const int row = lane >> 4, col = lane & 15, h = lane & 3;
  const int qhead0 = kvh * G;

  int seq = p.seq_lens[b];
  seq = max(0, min(seq, p.max_pages * kB));
  const int n_fin = summarized_pages(seq, p.pending);
  const int j0 = w * kExactPages;                          // first page of this workgroup
  const int n = max(0, min(kExactPages, n_fin - j0));     // its pages
  __shared__ __attribute__((aligned(16))) float outl[kSlots][kExactPages];
  float* __restrict__ lse_out = p.page_lse + ((size_t)b * p.hq + qhead0) * p.max_pages;

  // pages that are not finalized score -inf
  for (int j = n_fin + 64 * w + lane; j < p.max_pages; j += 64 * W)
#pragma unroll
    for (int hh = 0; hh < kSlots; ++hh)
      if (hh < G) lse_out[(size_t)hh * p.max_pages + j] = -INFINITY;
  if (n == 0) return;   // uniform: the whole (one-wave) workgroup leaves

  // slot 4 sub + h holds head 4 sub + h of the group (h % G when G < 4)
  bf16x8 bq[NSUB][4];
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    const int hs = 4 * sub + h;
    const uint16_t* qrow =
        p.q + ((size_t)b * p.hq + qhead0 + (hs < G ? hs : hs % G)) * kD + 32 * row;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      bq[sub][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 8 * s));
  }

  const int32_t* __restrict__ bt = p.block_table + (size_t)b * p.max_pages;
  const uint16_t* kbase = p.kc + (size_t)kvh * p.hs + (size_t)col * p.ts + 32 * row;
  // block id of step k; -1 for an out-of-range block id (block 0 is read, the
  // score dropped)
  auto bid_of = [&](int k) -> int {
    if (k >= n) return -1;
    const int x = bt[j0 + k];
    return ((unsigned)x < (unsigned)p.num_blocks) ? x : -1;
  };
  auto load = [&](int bid, uint4 kr[4]) {
    const uint16_t* kp = kbase + (size_t)max(bid, 0) * p.bs;
#pragma unroll
    for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const uint4*>(kp + 8 * s);
  };

  // software pipeline: keys two steps ahead, block ids three
  int b0 = bid_of(0), b1 = bid_of(1), b2 = bid_of(2);
  uint4 k0[4], k1[4];
  load(b0, k0);
  if (n > 1) load(b1, k1);
  for (int k = 0; k < n; ++k) {
    uint4 cur[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cur[s] = k0[s];
      k0[s] = k1[s];
    }
    const int bcur = b0;
    b0 = b1;
    b1 = b2;
    if (k + 2 < n) load(b1, k1);
    b2 = bid_of(k + 3);

    auto sub_pass = [&](const int sub) __attribute__((always_inline)) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) a = mfma16x16x32(as_bf16x8(cur[s]), bq[sub][s], a);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = a[r] * p.scale2;
      float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      m = cross_rows_max(m);
      float e = fast_exp2(x[0] - m) + fast_exp2(x[1] - m) + fast_exp2(x[2] - m) +
                fast_exp2(x[3] - m);
      e = cross_rows_sum(e);
      if (lane < 4) outl[4 * sub + h][k] = (bcur >= 0) ? (m + fast_log2(e)) * kLn2 : -INFINITY;
    };
    sub_pass(0);
    if constexpr (NSUB > 1) sub_pass(1);
  }
  // 4 lanes per head, 4 pages each
  __syncthreads();
  const int hh = lane >> 2, part = lane & 3;
  float* dst = lse_out + (size_t)hh * p.max_pages + j0 + 4 * part;
  const bool vec = (p.max_pages & 3) == 0 && ((uintptr_t)p.page_lse & 15) == 0;
  if (hh < G && 4 * part < n) {
    const float4 v = *reinterpret_cast<const float4*>(&outl[hh][4 * part]);
    if (vec && 4 * part + 4 <= n) {
      *reinterpret_cast<float4*>(dst) = v;
    } else {
      const float e[4] = {v.x, v.y, v.z, v.w};
      for (int i = 0; i < 4 && 4 * part + i < n; ++i) dst[i] = e[i];
    }
  }
}

}  // namespace

hipError_t launch_exact_lse(const uint16_t* q, const uint16_t* k_cache, int64_t block_stride,
                            int64_t head_stride, int64_t token_stride, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                            int32_t pending, float scale, float* page_lse, hipStream_t stream) {
  // kExactPages pages per wave: many short waves keep the end-of-launch tail small
  const int32_t W = std::max(1, (max_pages + kExactPages - 1) / kExactPages);
  const int32_t group = hq / hkv;
  ExactParams p{q, k_cache, block_stride, head_stride, token_stride, block_table, seq_lens,
                page_lse, scale * kLog2e, num_blocks, max_pages, hq, hkv, W, group, pending};
  if (group > 4)
    hipLaunchKernelGGL(exact_lse_kernel<2>, dim3(W, hkv, batch), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(exact_lse_kernel<1>, dim3(W, hkv, batch), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
