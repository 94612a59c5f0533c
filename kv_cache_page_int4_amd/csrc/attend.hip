// Sparse decode attention over the selected pages (LOCKS abstract: attend only
// the top pages; technical summary sec. 2: every query head of a GQA group
// attends the same page set).
//
// Split-K: the attended page list of a (sequence, KV head) -- the selected
// pages in ascending order, then the tail page (the tokens after the
// summarized pages, attended in full) -- is cut into splits
// of `pages_per_split` pages, one workgroup of 4 waves each; the waves take
// the split's pages in turn (wave w every 4th from the w-th), stream them
// page by page through LDS (see attend_wave) and merge their results in LDS
// into one partial per split.  Workgroups of 4 waves are dispatched 4 times
// faster than single waves, and the interleaving gives the waves of a split
// equal shares.  The query heads of the group share every K/V load.  A
// second kernel merges the splits by log-sum-exp into bf16 output.
#include "locks_device.h"
#include "locks_internal.h"
#include "select_common.h"

#include <algorithm>

namespace locks {

namespace {

constexpr int kWaves = 4;
constexpr long long kAttendWgs = 512;   // target workgroups (splits) per launch

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
  int32_t ntab;   // selection tables per sequence; KV head kvh reads table kvh / (hkv / ntab)
  int32_t group;  // query heads per KV head (1, 2, 4 or 8)
  int32_t pending;  // 1: the page holding the newest token is not summarized
};

// Global -> LDS copy of 16 bytes per lane: lane l writes LDS bytes
// [lds + 16 l, +16) from sbase + voff.  M0 carries the LDS address.  M0 is a
// register the compiler reserves, so listing it as clobbered is only a note
// to the reader (the compiler warns that it does not act on it): what makes
// this safe is that nothing else in these kernels uses M0 -- the generated
// code writes M0 only here, right before each copy.
// The copy is non-temporal: each K/V page is read once per step, and
// streaming it past the cache's normal allocation raises the read rate
// (each instruction reads one contiguous kilobyte, so no line is split
// between instructions).
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff),
               "s"(sbase), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int kPageBytes = 2 * kB * kD * 2;   // K then V of one page-head, bf16
constexpr int kAttRing = 2;                    // LDS page slots per wave: 1 in flight
constexpr int kRingBytes = kAttRing * kPageBytes;

// One wave's share of the attended page list of (sequence b, KV head kvh):
// the list is the first `count` entries of `selrow` (logical pages,
// ascending; nullptr means pages 0..count-1) and then the tail page;
// the wave takes its entries e_first, e_first + stride, ... (n_mine of
// them).  `selrow` may point to global memory or to LDS.  `ring` is this
// wave's LDS (kRingBytes); when the wave is done it holds the wave's
// unnormalized output and its (max, sum) per head slot (see wave_result),
// for the workgroup's merge.
//
// The split's block ids and token counts are resolved 64 pages at a time, one
// page per lane.  Each page-head's keys and values (8 KB) are then copied straight from
// HBM into an LDS slot with global->LDS DMA (8 instructions of 64 x 16 B),
// one page ahead of the one being computed (the ring depth less one).  The compiler does not
// track these copies: every page issues exactly 8, they complete in order,
// and a wait for "at most 8n outstanding" with n younger pages issued means
// this page has landed.  Any other memory instruction only makes it stricter.
//  * QK^T on the matrix cores: rows = the 16 tokens, K = head dim, columns =
//    4 query heads repeated 4 times; lane l gets tokens 4*(l/16)+r
//    (r = 0..3) of head slot l%4.  NSUB such 4-head sub-passes cover the
//    group: 2 for a group of 8 heads; a group of 1 or 2 fills the 4 slots
//    with its heads repeated (the duplicate slots are computed and dropped).
//  * online softmax in base 2 per page.
//  * P.V on the vector units: lane l keeps the same 4 tokens and dims
//    8*(l%16)..+8; the 4 slots' probabilities come from its quad by DPP.
template <int NSUB>
__device__ __forceinline__ void attend_wave(const AttendParams& p, int kvh, int b, int count,
                                            const int32_t* selrow, uint8_t* ring, int e_first,
                                            int stride, int n_mine) {
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, col = lane & 15, h = lane & 3;
  const int G = p.group;
  const int qhead0 = kvh * G;
  int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
  const int n_fin = summarized_pages(seq, p.pending);
  const int tail = seq - n_fin * kB;   // tokens attended in full (up to 16)
  const int n = n_mine;

  float M[NSUB], lsum[NSUB];
  float acc[NSUB][4][8];
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    M[sub] = -INFINITY;
    lsum[sub] = 0.f;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[sub][hh][e] = 0.f;
  }

  if (n > 0) {
    // slot 4 sub + h holds head 4 sub + h of the group (h % G when G < 4)
    uint4 qv[NSUB][4];
    bf16x8 bq[NSUB][4];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int hs = 4 * sub + h;
      const uint16_t* qrow =
          p.q + ((size_t)b * p.hq + qhead0 + (hs < G ? hs : hs % G)) * kD + 32 * row;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qv[sub][s] = *reinterpret_cast<const uint4*>(qrow + 8 * s);
        bq[sub][s] = as_bf16x8(qv[sub][s]);
      }
    }
    // unit u = 64 i + lane of a 4 KB half lands at LDS token u / 16, 16-byte
    // part u % 16.  Keys are stored XOR-swizzled (part c of token t holds the
    // key's part c ^ t), so that the 16 lanes reading one part of 16 tokens
    // hit 16 different banks; values are stored as they are.
    uint32_t voffk[4], voffv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = 64 * i + lane, t = u >> 4, c = u & 15;
      voffk[i] = (uint32_t)(t * p.ts * 2 + (c ^ t) * 16);
      voffv[i] = (uint32_t)(t * p.ts * 2 + c * 16);
    }
    const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    // chunks of up to 64 pages: block id and valid tokens of the wave's page
    // c0 + lane (list entry e_first + (c0 + lane) * stride) in lane `lane`
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int nc = min(64, n - c0);
      int mbid = 0, mnt = 0;
      if (lane < nc) {
        const int e = e_first + (c0 + lane) * stride;
        int j, nt;
        if (e < count) {
          j = selrow ? selrow[e] : e;
          nt = (j >= 0 && j < n_fin) ? kB : 0;
        } else {
          j = n_fin;
          nt = tail;
        }
        int bid = (nt > 0) ? bt[j] : 0;
        if ((unsigned)bid >= (unsigned)p.num_blocks) {
          bid = 0;
          nt = 0;
        }
        mbid = bid;
        mnt = nt;
      }
      // consume the loads above here, so that the compiler's waits for them
      // come before the first page copies are issued
      asm volatile("" ::"v"(mbid), "v"(mnt), "v"(qv[0][0].x), "v"(qv[0][1].x), "v"(qv[0][2].x),
                   "v"(qv[0][3].x));
      if constexpr (NSUB > 1)
        asm volatile("" ::"v"(qv[NSUB - 1][0].x), "v"(qv[NSUB - 1][1].x),
                     "v"(qv[NSUB - 1][2].x), "v"(qv[NSUB - 1][3].x));
      auto issue = [&](int k) {
        const int bid = __builtin_amdgcn_readlane(mbid, k);
        const uint16_t* kb = p.kc + (size_t)bid * p.bs + (size_t)kvh * p.hs;
        const uint16_t* vb = p.vc + (size_t)bid * p.bs + (size_t)kvh * p.hs;
        const uint32_t slot = ring0 + (uint32_t)((k % kAttRing) * kPageBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(voffk[i], kb, __builtin_amdgcn_readfirstlane(slot + 1024 * i));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16(voffv[i], vb, __builtin_amdgcn_readfirstlane(slot + 4096 + 1024 * i));
      };

      wait_lgkm0();   // the previous chunk's last LDS reads
      for (int k = 0; k < kAttRing - 1 && k < nc; ++k) issue(k);
      for (int k = 0; k < nc; ++k) {
        // every LDS read of page k-1 has returned: its slot may be refilled
        wait_lgkm0();
        if (k + kAttRing - 1 < nc) issue(k + kAttRing - 1);
        const int ahead = min(kAttRing - 1, nc - 1 - k);   // younger pages in flight
        static_assert(kAttRing <= 4, "wait counts below cover at most 3 pages ahead");
        if (ahead >= 3) wait_vm<24>();
        else if (ahead == 2) wait_vm<16>();
        else if (ahead == 1) wait_vm<8>();
        else wait_vm<0>();
        const uint8_t* S = ring + (k % kAttRing) * kPageBytes;
        const int ntok = __builtin_amdgcn_readlane(mnt, k);
        // ---- logits of tokens 4 row + r for head slot col % 4 ----
        float P[NSUB][4];
        auto logits = [&](const int sub) __attribute__((always_inline)) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint4 kv = *reinterpret_cast<const uint4*>(S + col * 256 + 16 * ((4 * row + s) ^ col));
            a = mfma16x16x32(as_bf16x8(kv), bq[sub][s], a);
          }
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = (4 * row + r < ntok) ? a[r] * p.scale2 : -INFINITY;
          float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
          mx = cross_rows_max(mx);
          const float Mn = fmaxf(M[sub], mx);
          const float alpha = (Mn == -INFINITY) ? 1.f : fast_exp2(M[sub] - Mn);
          float ps = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            P[sub][r] = (x[r] == -INFINITY) ? 0.f : fast_exp2(x[r] - Mn);
            ps += P[sub][r];
          }
          lsum[sub] = lsum[sub] * alpha + ps;
          M[sub] = Mn;
          const float al[4] = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha),
                               quad_bcast<3>(alpha)};
#pragma unroll
          for (int hh = 0; hh < 4; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[sub][hh][e] *= al[hh];
        };
        logits(0);
        if constexpr (NSUB > 1) logits(1);
        // ---- P.V: tokens 4 row + r, dims 8 col .. 8 col + 7, all head slots ----
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint4 v = *reinterpret_cast<const uint4*>(S + 4096 + (4 * row + r) * 256 + 16 * col);
          const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                               bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
          auto pv = [&](const int sub) __attribute__((always_inline)) {
            const float p0 = quad_bcast<0>(P[sub][r]), p1 = quad_bcast<1>(P[sub][r]);
            const float p2 = quad_bcast<2>(P[sub][r]), p3 = quad_bcast<3>(P[sub][r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              acc[sub][0][e] = fmaf(p0, vf[e], acc[sub][0][e]);
              acc[sub][1][e] = fmaf(p1, vf[e], acc[sub][1][e]);
              acc[sub][2][e] = fmaf(p2, vf[e], acc[sub][2][e]);
              acc[sub][3][e] = fmaf(p3, vf[e], acc[sub][3][e]);
            }
          };
          pv(0);
          if constexpr (NSUB > 1) pv(1);
        }
      }
    }
  }
  // each row of lanes holds a quarter of the tokens: sum the rows
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[sub][hh][e] = cross_rows_sum(acc[sub][hh][e]);
    lsum[sub] = cross_rows_sum(lsum[sub]);
  }
  // the wave's result into its own ring (every copy into it has landed and
  // every read of it has returned): wave_result layout
  wait_lgkm0();
  float* res = reinterpret_cast<float*>(ring);
  if (row == 0) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        float* o = res + (4 * sub + hh) * kD + 8 * col;
        *reinterpret_cast<float4*>(o) =
            make_float4(acc[sub][hh][0], acc[sub][hh][1], acc[sub][hh][2], acc[sub][hh][3]);
        *reinterpret_cast<float4*>(o + 4) =
            make_float4(acc[sub][hh][4], acc[sub][hh][5], acc[sub][hh][6], acc[sub][hh][7]);
      }
      if (col < 4) {
        res[4 * NSUB * kD + 2 * (4 * sub + col)] = M[sub];
        res[4 * NSUB * kD + 2 * (4 * sub + col) + 1] = lsum[sub];
      }
    }
  }
}

// The kWaves waves of a workgroup took interleaved entries of one split of
// the attended page list; each left its (unnormalized output, max, sum) per
// head slot in its ring (floats: [slot][128] then (max, sum) per slot).
// After a barrier the workgroup merges them by log-sum-exp into one partial
// per real head and split: thread t of the first 256 takes head slot
// t / 64 (+ 4 per pass) and dims 2 (t % 64), +1.
template <int NSUB>
__device__ __forceinline__ void wg_merge_store(const AttendParams& p, int split, int kvh, int b,
                                               const uint8_t* rings) {
  const int t = threadIdx.x;
  if (t >= 64 * kWaves) return;
  const int G = p.group;
  const int qhead0 = kvh * G;
  const int d0 = 2 * (t & 63);
#pragma unroll
  for (int pass = 0; pass < NSUB; ++pass) {
    const int slot = 4 * pass + (t >> 6);
    if (slot >= G) continue;   // a repeated head slot
    float Mw[kWaves], Lw[kWaves];
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* res = reinterpret_cast<const float*>(rings + w * kRingBytes);
      Mw[w] = res[4 * NSUB * kD + 2 * slot];
      Lw[w] = res[4 * NSUB * kD + 2 * slot + 1];
      Mx = fmaxf(Mx, Mw[w]);
    }
    float o0 = 0.f, o1 = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* res = reinterpret_cast<const float*>(rings + w * kRingBytes);
      const float sc = (Mw[w] == -INFINITY) ? 0.f : fast_exp2(Mw[w] - Mx);
      const float2 v = *reinterpret_cast<const float2*>(res + slot * kD + d0);
      o0 = fmaf(sc, v.x, o0);
      o1 = fmaf(sc, v.y, o1);
      l = fmaf(sc, Lw[w], l);
    }
    const size_t prow = ((size_t)b * p.hq + qhead0 + slot) * p.n_splits + split;
    *reinterpret_cast<float2*>(p.part_o + prow * kD + d0) = make_float2(o0, o1);
    if ((t & 63) == 0) p.part_ml[prow] = make_float2(Mx, l);
  }
}

// The waves' entries of split `split` of a list of n_att entries: wave w of
// the workgroup takes entries base + w, base + w + kWaves, ... below the
// split's end.
__device__ __forceinline__ void split_share(const AttendParams& p, int split, int n_att, int wave,
                                            int* e_first, int* n_mine) {
  const int base = split * p.pages_per_split;
  const int end = min(base + p.pages_per_split, n_att);
  *e_first = base + wave;
  *n_mine = (*e_first < end) ? (end - *e_first + kWaves - 1) / kWaves : 0;
}

__device__ __forceinline__ int attended_entries(const AttendParams& p, int b, int count) {
  const int seq = max(0, min(p.seq_lens[b], p.max_pages * kB));
  return count + (seq > summarized_pages(seq, p.pending) * kB ? 1 : 0);
}

// kWaves waves per workgroup, one split each, 16 KB of LDS per wave: two
// workgroups (eight waves) share a CU.
template <int NSUB>
__global__ __launch_bounds__(64 * kWaves) void attend_kernel(AttendParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kRingBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  int count;
  const int32_t* selrow = nullptr;
  if (p.sel) {
    const size_t tab = (size_t)b * p.ntab + kvh / (p.hkv / p.ntab);
    count = max(0, min(p.sel_count[tab], p.budget));
    selrow = p.sel + tab * p.budget;
  } else {
    count = summarized_pages(max(0, min(p.seq_lens[b], p.max_pages * kB)), p.pending);
  }
  int e_first, n_mine;
  split_share(p, split, attended_entries(p, b, count), wave, &e_first, &n_mine);
  attend_wave<NSUB>(p, kvh, b, count, selrow, &ring[wave][0], e_first, kWaves, n_mine);
  __syncthreads();
  wg_merge_store<NSUB>(p, split, kvh, b, &ring[0][0]);
}

// ---- final selection fused with the attention --------------------------------
// Every workgroup of a (sequence, KV head) runs the last selection stage of
// its table itself (the top k of that table's chunk candidates, 256 threads),
// keeps the ascending page list in LDS and attends its splits from there: no
// kernel boundary and no global round trip between choosing the pages and
// reading them.  The selection is the same computation as the stand-alone
// stage, on the same candidates in the same order, so its result is
// identical; workgroup 0 of the table's first KV head also writes it out.
struct FusedSel {
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  int32_t* sel;
  int32_t* sel_count;
  int32_t n_chunks, slots;
};

constexpr int kFusedThreads = 256;
constexpr long long kFusedWideGrid = 256;   // fused workgroups up to which 1024 threads select

// NT threads run the selection (NT = 1024 when the grid leaves a CU per
// workgroup: four candidates per thread instead of sixteen at 1M); the first
// kWaves waves then attend and the others leave.
template <int RUN, int NT, int NSUB>
__global__ __launch_bounds__(NT) void select_attend_kernel(AttendParams p, FusedSel f) {
  constexpr int kFusedThreads = NT;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  __shared__ int hist[2][256];
  __shared__ int sh[2][4];
  __shared__ uint32_t red_smem[3 * (kFusedThreads / 64)];
  __shared__ int scan_smem[kFusedThreads / 64];
  __shared__ int32_t sel_lds[kFusedMaxBudget];
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kRingBytes];

  const int n_cand = f.n_chunks * f.slots;
  const int kv_per_tab = p.hkv / p.ntab;
  const size_t grp = (size_t)b * p.ntab + kvh / kv_per_tab;   // this KV head's table
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
  if (blockIdx.x == 0 && kvh % kv_per_tab == 0) {   // one writer per table
    int32_t* out = f.sel + grp * p.budget;
    for (int s = tid; s < p.budget; s += kFusedThreads) out[s] = (s < k) ? sel_lds[s] : -1;
    if (tid == 0) f.sel_count[grp] = k;
  }
  // the first kWaves waves attend split blockIdx.x (interleaved entries) and
  // merge it; the others only pass the barrier
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int split = blockIdx.x;
  if (wave < kWaves) {
    int e_first, n_mine;
    split_share(p, split, attended_entries(p, b, k), wave, &e_first, &n_mine);
    attend_wave<NSUB>(p, kvh, b, k, sel_lds, &ring[wave][0], e_first, kWaves, n_mine);
  }
  __syncthreads();
  wg_merge_store<NSUB>(p, split, kvh, b, &ring[0][0]);
}

// One workgroup per (sequence, query head): log-sum-exp weights of the
// splits, then out[d] = sum_s w_s o_s[d] / sum_s w_s l_s.  Wave v takes the
// splits s = v (mod 4) with lane l owning dims 2l, 2l+1 (one 512 B row per
// split per wave), eight rows in flight per wave; the four wave sums meet in
// LDS.
constexpr int kMergeW = 4096;
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;

__global__ __launch_bounds__(kMergeThreads) void attend_merge_kernel(AttendParams p) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const size_t row = (size_t)b * p.hq + h;
  const int n = p.n_splits;
  const float2* ml = p.part_ml + row * n;
  __shared__ float wsh[kMergeW];
  __shared__ float red[kMergeWaves];
  __shared__ float2 accsh[kMergeWaves][64];
  float M = -INFINITY;
  for (int s = t; s < n; s += kMergeThreads) M = fmaxf(M, ml[s].x);
  M = wave_max_f(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  auto weight = [&](float m) { return (m == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(m - M); };
  float L = 0.f;
  for (int s = t; s < n; s += kMergeThreads) {
    const float2 v = ml[s];
    const float w = weight(v.x);
    if (s < kMergeW) wsh[s] = w;
    L += w * v.y;
  }
  L = wave_sum_f(L);
  if (lane == 0) red[wave] = L;
  __syncthreads();   // also publishes wsh
  L = red[0] + red[1] + red[2] + red[3];

  const float2* po = reinterpret_cast<const float2*>(p.part_o + row * n * kD) + lane;
  float2 acc = make_float2(0.f, 0.f);
  int s = wave;
  for (; s + 7 * kMergeWaves < n; s += 8 * kMergeWaves) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = po[(size_t)(s + u * kMergeWaves) * (kD / 2)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ss = s + u * kMergeWaves;
      const float w = (ss < kMergeW) ? wsh[ss] : weight(ml[ss].x);
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
    }
  }
  for (; s < n; s += kMergeWaves) {
    const float w = (s < kMergeW) ? wsh[s] : weight(ml[s].x);
    const float2 v = po[(size_t)s * (kD / 2)];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
  }
  accsh[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float2 r = accsh[0][lane];
#pragma unroll
    for (int v = 1; v < kMergeWaves; ++v) {
      r.x += accsh[v][lane].x;
      r.y += accsh[v][lane].y;
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    const uint32_t lo = f32_to_bf16(r.x * inv), hi = f32_to_bf16(r.y * inv);
    reinterpret_cast<uint32_t*>(p.out + row * kD)[lane] = lo | (hi << 16);
    if (p.out_lse && lane == 0) p.out_lse[row] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : -INFINITY;
  }
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
                                int32_t ntab, int32_t pending, const uint32_t* cand_key,
                                const int32_t* cand_idx, const SelectPlan& sp, int32_t* sel,
                                int32_t* sel_count, int32_t budget_pages, float scale,
                                float* part_o, float2* part_ml, const AttendPlan& plan,
                                uint16_t* out, float* out_lse, hipStream_t stream) {
  AttendParams p{q, k_cache, v_cache, block_stride, head_stride, token_stride, block_table,
                 seq_lens, sel, sel_count, part_o, part_ml, out, out_lse,
                 scale * kLog2e, num_blocks, max_pages, budget_pages, hq, hkv,
                 plan.pages_per_split, plan.n_splits, ntab, hq / hkv, pending};
  FusedSel f{cand_key, cand_idx, sel, sel_count, sp.n_chunks, sp.slots};
  const int32_t n_cand = sp.n_chunks * sp.slots;
  dim3 grid(plan.n_splits, hkv, batch);
  const long long wgs = (long long)grid.x * grid.y * grid.z;
  const bool two = p.group > 4;   // two 4-head sub-passes
#define LOCKS_SA(RUN, NT)                                                                     \
  do {                                                                                        \
    if (two)                                                                                  \
      hipLaunchKernelGGL((select_attend_kernel<RUN, NT, 2>), grid, dim3(NT), 0, stream, p, f); \
    else                                                                                      \
      hipLaunchKernelGGL((select_attend_kernel<RUN, NT, 1>), grid, dim3(NT), 0, stream, p, f); \
  } while (0)
  if (!two && wgs <= kFusedWideGrid && n_cand > 4 * kFusedThreads) {
    // one workgroup per CU at most: select with 1024 threads (a group of 8
    // heads needs more registers than 1024 threads leave, and keeps 256)
    const int per = (n_cand + 1023) / 1024;
    if (per <= 4)
      hipLaunchKernelGGL((select_attend_kernel<4, 1024, 1>), grid, dim3(1024), 0, stream, p, f);
    else
      hipLaunchKernelGGL((select_attend_kernel<8, 1024, 1>), grid, dim3(1024), 0, stream, p, f);
  } else {
    const int per = (n_cand + kFusedThreads - 1) / kFusedThreads;
    if (per <= 4) LOCKS_SA(4, kFusedThreads);
    else if (per <= 16) LOCKS_SA(16, kFusedThreads);
    else LOCKS_SA(32, kFusedThreads);
  }
#undef LOCKS_SA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(hq, batch), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

AttendPlan plan_attend(int32_t batch, int32_t hkv, int32_t max_attended) {
  // a split is one workgroup of kWaves waves: about kAttendWgs of them over
  // all (sequence, KV head) groups (two per CU, so that none waits for a
  // second round), at least two pages per wave
  AttendPlan pl;
  const long long groups = (long long)batch * hkv;
  const long long total = groups * (long long)max_attended;
  long long pages = (total + kAttendWgs - 1) / kAttendWgs;
  pages = std::max(2LL * kWaves, std::min(8192LL, pages));
  pl.pages_per_split = (int32_t)pages;
  pl.n_splits = (int32_t)((max_attended + pages - 1) / pages);
  if (pl.n_splits < 1) pl.n_splits = 1;
  return pl;
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         int64_t block_stride, int64_t head_stride, int64_t token_stride,
                         int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                         const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                         int32_t ntab, int32_t pending, const int32_t* sel,
                         const int32_t* sel_count, int32_t budget_pages, float scale,
                         float* part_o, float2* part_ml, const AttendPlan& plan, uint16_t* out,
                         float* out_lse, hipStream_t stream) {
  AttendParams p{q, k_cache, v_cache, block_stride, head_stride, token_stride, block_table,
                 seq_lens, sel, sel_count, part_o, part_ml, out, out_lse,
                 scale * kLog2e, num_blocks, max_pages, budget_pages, hq, hkv,
                 plan.pages_per_split, plan.n_splits, ntab, hq / hkv, pending};
  dim3 grid(plan.n_splits, hkv, batch);
  if (p.group > 4)
    hipLaunchKernelGGL(attend_kernel<2>, grid, dim3(64 * kWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(attend_kernel<1>, grid, dim3(64 * kWaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3(hq, batch), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
