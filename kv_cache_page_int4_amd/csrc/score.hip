// Page scoring from summaries: s_hat_j(q) = LSE_i((q.mu_j + (V_j^T q).c_i)/sqrt(d))
// (LOCKS explainer, technical summary sec. 2, reconstruction and selection).
//
// Work split.  The pages of one (sequence, KV head) are cut into 4-page
// steps.  Workgroup g of a (sequence, KV head) has kScoreWaves independent
// waves; wave v takes the kScoreSteps consecutive steps from
// (g * kScoreWaves + v) * kScoreSteps on, so the workgroup covers one
// contiguous run of pages.  Waves are short: many dispatch rounds keep the
// end-of-launch tail small.  The page LSEs of all waves are collected in LDS
// and leave at the end as one contiguous run per head (256 bytes, two whole
// lines), and the waves' (max, sum) partials are merged into one per head.
// Stores are few on purpose: under a full HBM read stream every store
// instruction, even a whole-line one, costs far more time than its bytes.
//
// Data movement.  The four 832-byte records of a step are copied straight
// from HBM into the wave's LDS slot with global->LDS DMA (one 816-byte
// instruction per record: 51 lanes x 16 B; the trailing pad is skipped),
// marked non-temporal: the records are read once, and streaming them past
// the cache's normal allocation raises the read rate.  One slot per wave:
// the step's LDS reads all complete (into registers) before the next step's
// copies are issued into the same slot, and those copies are in flight while
// the step computes.  The group's query heads sit in LDS too, so a wave holds
// no q in VGPRs; with 4.3 KB of LDS and at most 72 VGPRs per wave, seven
// waves share each SIMD.  The compiler does not track these copies, so the
// issue and the waits are written out: a step is the only copy in flight when
// it is waited for, so waiting for zero outstanding means it has landed.
//
// GQA groups of G = 1, 2, 4 or 8 query heads.  The matrix-core tiles below
// have 4 head columns (each repeated 4 times); a group of 8 runs the per-step
// arithmetic twice on the same LDS-resident records (two 4-head sub-passes),
// and a group of 1 or 2 fills the 4 columns with its heads repeated (the
// duplicate columns are computed and dropped).
//
// Per step one wave does (for each 4-head sub-pass):
//  * V^T q on the matrix cores: rows = (page, basis) pairs, K = head dim,
//    columns = 4 query heads of the group repeated 4 times.  The int4
//    basis codes become bf16 values 136+n exactly (byte permute onto the
//    exponent of 128); the accumulator starts at -136*sum(q).  With the
//    rows ordered (page = lane/16, basis = register), lane l ends up holding
//    w[page l/16][k][head l%4] for all 8 k.
//  * q.mu on the matrix cores: rows (page p, dim group s''), columns
//    (dim group s', head h), K over the 4 dim quarters; the diagonal
//    s'' = s' summed over s' is q_h.mu_p.  Lane l picks its diagonal entry
//    and the 4 lanes 4 apart in the row add up the rest.
//  * the coefficient term on the matrix cores, one 16-block 4x4x1 fp32
//    MFMA per basis index: lane l keeps its own head h = l%4 and page l/16
//    and gets the 4 tokens 4*cg..4*cg+3 of that page (cg = (l%16)/4).
//  * the page LSE over 16 tokens: 4 exponentials in the lane, then the 4
//    lanes of the same (page, head) -- 4 and 8 apart in the row -- are summed
//    with two DPP row rotations.
#include "locks_device.h"
#include "locks_internal.h"

#include <algorithm>

namespace locks {

namespace {

constexpr uint32_t kMagic = 0x43434343u;  // bf16 high byte of 128.0
constexpr int kScoreWaves = 4;            // independent waves per workgroup

// 8 int4 codes (two's complement, layout of the record) -> 8 bf16 = 136 + code.
__device__ __forceinline__ bf16x8 nib8_to_bf16(uint32_t x) {
  x ^= 0x88888888u;                       // code + 8 in [1, 15]
  const uint32_t lo = x & 0x0F0F0F0Fu;    // dims 0..3 of the word, one per byte
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // dims 4..7
  uint4 w;
  w.x = __builtin_amdgcn_perm(kMagic, lo, 0x04010400u);
  w.y = __builtin_amdgcn_perm(kMagic, lo, 0x04030402u);
  w.z = __builtin_amdgcn_perm(kMagic, hi, 0x04010400u);
  w.w = __builtin_amdgcn_perm(kMagic, hi, 0x04030402u);
  return as_bf16x8(w);
}

// 8 int8 codes -> 8 exact bf16 values.
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint2 v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(float)(int8_t)(v.x >> (8 * e));
    r[4 + e] = (__bf16)(float)(int8_t)(v.y >> (8 * e));
  }
  return r;
}


// Field offsets of a rank-R record (the rank-8 layout with every field sized
// by R) and its LDS slot: the record's fields are copied in whole 16-byte
// units, the trailing pad skipped (51 units at rank 8), one or two DMA
// instructions per record.
template <int R>
struct ScoreLayout {
  static constexpr int kRecB = rec_bytes(R);
  static constexpr int kOffC = 64 * R, kOffMu = 80 * R, kOffSv = 80 * R + 128;
  static constexpr int kOffSc = 82 * R + 128, kOffSmu = 84 * R + 128;
  static constexpr int kUnits = (84 * R + 130 + 15) / 16;
  static constexpr int kSlotRec = 16 * kUnits;
  static constexpr int kStepBytes = 4 * kSlotRec;
  static constexpr int kDmaPerRec = (kUnits + 63) / 64;
};

struct ScoreParams {
  const uint16_t* q;
  const uint8_t* summ;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* page_lse;
  float2* partials;
  float c0;   // logit scale times log2(e): base-2 logits
  int32_t num_blocks, max_pages, hq, hkv, n_wg;
  int32_t group;   // query heads per KV head (1, 2, 4 or 8)
  int32_t pending; // 1: the page holding the newest token is not summarized
};

// Global -> LDS copy of 16 bytes per active lane: lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16) from sbase + voff.  M0 carries the LDS
// address.  M0 is a register the compiler reserves, so listing it as
// clobbered is only a note to the reader (the compiler warns that it does not
// act on it): what makes this safe is that nothing else in the kernel uses
// M0 -- the generated code writes M0 only here, right before each copy.
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

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// NSUB: 4-head sub-passes per step (2 for a group of 8 heads, else 1).
// Waves per SIMD the register budget is cut for: 7 (at most 72 registers)
// for one head pass at ranks 4 and 8; rank 16 needs 96 registers for one
// pass (5 waves); a group of 8 heads at rank 8 needs a little more than 96
// registers and is held to 96 (5 waves instead of 4).
constexpr int score_waves(int r, int nsub) {
  return nsub == 1 ? (r == 16 ? 5 : 7) : (r == 4 ? 7 : (r == 8 ? 5 : 3));
}

template <int R, int NSUB>
__global__ __launch_bounds__(64 * kScoreWaves) __attribute__((
    amdgpu_waves_per_eu(score_waves(R, NSUB), score_waves(R, NSUB)))) void
score_kernel(ScoreParams p) {
  using SL = ScoreLayout<R>;
  constexpr int kSlotRec = SL::kSlotRec, kStepBytes = SL::kStepBytes;
  constexpr int kOffC = SL::kOffC, kOffMu = SL::kOffMu, kOffSv = SL::kOffSv;
  constexpr int kOffSc = SL::kOffSc, kOffSmu = SL::kOffSmu;
  constexpr int kWavePages = 4 * kScoreSteps;             // pages of one wave
  constexpr int kWgPages = kScoreWaves * kWavePages;       // pages of the workgroup
  __shared__ __attribute__((aligned(16))) uint8_t ring_all[kScoreWaves][kStepBytes];
  constexpr int kSlots = 4 * NSUB;   // head slots: 4 per sub-pass
  __shared__ __attribute__((aligned(16))) uint4 qs_all[kScoreWaves][kSlots * kD / 8];
  __shared__ __attribute__((aligned(16))) float outl[kSlots][kWgPages];
  __shared__ float2 red[kScoreWaves][kSlots];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave in the workgroup
  uint8_t* ring = ring_all[wv];          // this wave's record slot
  uint4* qs = qs_all[wv];                // this wave's copy of the group's query heads
  const int g = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int W = p.n_wg;
  const int G = p.group;
  const int qhead0 = kvh * G;
  const int row = lane >> 4;   // page slot of this lane in a step
  const int tok = lane & 15;
  const int h = lane & 3;      // head slot of this lane within a sub-pass

  int seq = p.seq_lens[b];
  seq = max(0, min(seq, p.max_pages * kB));
  const int n_fin = summarized_pages(seq, p.pending);
  const int nsteps = (n_fin + 3) / 4;
  const int s0 = (g * kScoreWaves + wv) * kScoreSteps;    // first step of this wave
  const int n = max(0, min(kScoreSteps, nsteps - s0));    // its steps

  const uint8_t* __restrict__ summ_h = p.summ + (size_t)kvh * p.num_blocks * SL::kRecB;
  const int32_t* __restrict__ bt = p.block_table + (size_t)b * p.max_pages;
  float* __restrict__ lse_out = p.page_lse + ((size_t)b * p.hq + qhead0) * p.max_pages;

  // pages that are not finalized score -inf (each written once: a grid-stride
  // loop over all threads of the (sequence, KV head)'s workgroups)
  constexpr int kThreads = 64 * kScoreWaves;
  for (int j = n_fin + kThreads * g + (int)threadIdx.x; j < p.max_pages; j += kThreads * W)
    for (int hh = 0; hh < G; ++hh) lse_out[(size_t)hh * p.max_pages + j] = -INFINITY;

  // running base-2 (max, sum) of head slot 4 sub + h (lanes tok < 4)
  float pm[NSUB], ps[NSUB];
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    pm[sub] = -INFINITY;
    ps[sub] = 0.f;
  }
  if (n > 0) {
    // The group's query heads (1 KB of bf16 per sub-pass) are staged in LDS
    // once and each step reads its MFMA B operands from there, which keeps
    // them out of VGPRs.  Slot hs holds head hs of the group (head hs % G
    // when G < 4).  For V^T q, column (lane%16) is slot lane%4 of the
    // sub-pass and K element (step s, lane group g, e) is dim 32g + 8s + e.
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const int u = 64 * i + lane, hs = u >> 4;
      const int src = qhead0 + (hs < G ? hs : hs % G);
      qs[u] = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.hq + src) * kD + 8 * (u & 15));
    }
    auto qpiece = [&](int sub, int s) -> uint4 { return qs[(4 * sub + h) * (kD / 8) + 4 * row + s]; };
    // the codes enter the product as 136 + n: start the accumulator at -136 sum(q)
    float acc0_init[NSUB];
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      float qsum = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 v = qpiece(sub, s);
        qsum += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
                bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
      }
      acc0_init[sub] = -136.f * cross_rows_sum(qsum);
    }
    // for q.mu, column (lane%16) = (dim group s' = (lane/4)%4, slot lane%4) and
    // K element (lane group g, e) is dim 32g + 8s' + e
    const int sq = (lane >> 2) & 3;
    const float c0 = p.c0;   // base-2 logit scale

    const uint32_t ring0 =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[0];
    // block ids of step k (scalar loads through the constant address space);
    // -1 marks a page past the finalized ones or with an out-of-range block id
    // (its record 0 is copied and its score dropped)
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;
    auto step_bids = [&](int k) -> int4 {
      const int j0 = 4 * (s0 + k);
      const unsigned nbk = (unsigned)p.num_blocks;
      int4 v;
      if (j0 + 4 <= n_fin) {
        v.x = btc[j0];
        v.y = btc[j0 + 1];
        v.z = btc[j0 + 2];
        v.w = btc[j0 + 3];
      } else {
        v.x = btc[min(j0, n_fin - 1)];
        v.y = (j0 + 1 < n_fin) ? btc[j0 + 1] : -1;
        v.z = (j0 + 2 < n_fin) ? btc[j0 + 2] : -1;
        v.w = (j0 + 3 < n_fin) ? btc[j0 + 3] : -1;
      }
      v.x = ((unsigned)v.x < nbk) ? v.x : -1;
      v.y = ((unsigned)v.y < nbk) ? v.y : -1;
      v.z = ((unsigned)v.z < nbk) ? v.z : -1;
      v.w = ((unsigned)v.w < nbk) ? v.w : -1;
      return v;
    };
    auto issue = [&](int4 bb) {
      const uint32_t slot = ring0;
      const int bi[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* base = summ_h + (size_t)max(bi[i], 0) * SL::kRecB;
#pragma unroll
        for (int u = 0; u < SL::kDmaPerRec; ++u)
          if (64 * u + lane < SL::kUnits)
            dma16(16u * (64 * u + lane), base,
                  __builtin_amdgcn_readfirstlane(slot + kSlotRec * i + 1024 * u));
      }
    };

    // block ids of step k (b0) and k+1 (b1, the next one to issue)
    const int4 none = make_int4(-1, -1, -1, -1);
    int4 b0 = step_bids(0);
    int4 b1 = (n > 1) ? step_bids(1) : none;
    issue(b0);
    for (int k = 0; k < n; ++k) {
      const int4 bcur = b0;
      const bool more = k + 1 < n;
      // step k is the only copy in flight
      wait_vm<0>();

      const uint8_t* S = &ring[0];
      const uint8_t* Sr = S + kSlotRec * row;          // record of this lane's page
      const int jpg = 4 * (s0 + k) + row;              // this lane's page
      const int bid_row = (row == 0) ? bcur.x : (row == 1) ? bcur.y : (row == 2) ? bcur.z : bcur.w;
      const bool okp = bid_row >= 0;

      // ---- every LDS read of the step; then the slot takes step k+1 ----
      constexpr int kAcc = R / 4;   // V^T q accumulators: basis columns 4j .. 4j+3
      // basis codes: A rows (page tok/4, basis tok%4 + 4j), dims 32 row + 8s + e
      const uint8_t* av = S + kSlotRec * (tok >> 2) + 64 * (lane & 3) + 16 * row;
      uint4 va[kAcc];
#pragma unroll
      for (int j = 0; j < kAcc; ++j) va[j] = lds16(av + 256 * j);
      // centroid codes: A row (page (lane/4)%4, dim group lane%4), K (lane group g, e)
      const uint2 mq = *reinterpret_cast<const uint2*>(S + kSlotRec * sq + kOffMu + 32 * row +
                                                       8 * (lane & 3));
      const uint16_t smu_raw = *reinterpret_cast<const uint16_t*>(Sr + kOffSmu);
      uint32_t svw[R / 2], scw[R / 2];
#pragma unroll
      for (int i = 0; i < R / 2; ++i) {
        svw[i] = *reinterpret_cast<const uint32_t*>(Sr + kOffSv + 4 * i);
        scw[i] = *reinterpret_cast<const uint32_t*>(Sr + kOffSc + 4 * i);
      }
      // coefficient codes of this lane's token
      const uint8_t* cp = Sr + kOffC + R * tok;
      uint32_t cw[R / 4];
      if constexpr (R == 4) {
        cw[0] = *reinterpret_cast<const uint32_t*>(cp);
      } else if constexpr (R == 8) {
        const uint2 c2 = *reinterpret_cast<const uint2*>(cp);
        cw[0] = c2.x;
        cw[1] = c2.y;
      } else {
        const uint4 c4 = lds16(cp);
        cw[0] = c4.x;
        cw[1] = c4.y;
        cw[2] = c4.z;
        cw[3] = c4.w;
      }
      wait_lgkm0();
      if (more) issue(b1);
      b0 = b1;
      b1 = (k + 2 < n) ? step_bids(k + 2) : none;

      auto sub_pass = [&](const int sub) __attribute__((always_inline)) {
        // ---- V^T q on the matrix cores ----
        f32x4 acc[kAcc];
        const float a0 = acc0_init[sub];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = f32x4{a0, a0, a0, a0};
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
          acc[j] = mfma16x16x32(nib8_to_bf16(va[j].x), as_bf16x8(qpiece(sub, 0)), acc[j]);
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
          acc[j] = mfma16x16x32(nib8_to_bf16(va[j].y), as_bf16x8(qpiece(sub, 1)), acc[j]);
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
          acc[j] = mfma16x16x32(nib8_to_bf16(va[j].z), as_bf16x8(qpiece(sub, 2)), acc[j]);
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
          acc[j] = mfma16x16x32(nib8_to_bf16(va[j].w), as_bf16x8(qpiece(sub, 3)), acc[j]);

        // ---- q.mu ----
        f32x4 dmu = {0.f, 0.f, 0.f, 0.f};
        dmu = mfma16x16x32(i8x8_to_bf16(mq), as_bf16x8(qpiece(sub, sq)), dmu);
        // lane (page row, s' = sq, slot h) holds D[(row, r)][(sq, h)] in register r
        float qmu = (sq == 0) ? dmu[0] : (sq == 1) ? dmu[1] : (sq == 2) ? dmu[2] : dmu[3];
        qmu += dpp<kRowRor4>(qmu);
        qmu += dpp<kRowRor8>(qmu);
        const float qmu2 = qmu * half_lo(smu_raw) * c0;

        // ---- w[k] = (q_h.v_k) * s_V[k] * s_c[k] for this lane's page and head ----
        // fp16 operand times fp32 with a +0 addend: one mixed-precision FMA each
        auto hmul = [](uint32_t pair, int hi, float x) {
          return __builtin_fmaf(hi ? half_hi(pair) : half_lo(pair), x, 0.0f);
        };
        float wk[R];
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kk = 4 * j + r;
            wk[kk] = hmul(scw[kk >> 1], kk & 1, hmul(svw[kk >> 1], kk & 1, acc[j][r]));
          }
        // ---- deviation logits (base 2, without q.mu) of tokens 4cg..4cg+3 ----
        // One 16-block 4x4x1 MFMA per basis index k: block l/4 is (page, token
        // quarter cg), its rows the 4 tokens, its columns the 4 head slots.
        // Lane l gives A = c[token l%16][k] and B = w[k] of its own page and
        // slot; it gets back tokens 4cg..4cg+3 of slot l%4.  Each code is
        // converted once instead of once per head, and the products stay fp32.
        f32x4 dv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < R; ++kk)
          dv = __builtin_amdgcn_mfma_f32_4x4x1f32((float)(int8_t)(cw[kk >> 2] >> (8 * (kk & 3))),
                                                  wk[kk], dv, 0, 0, 0);
        float dl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) dl[t] = dv[t] * c0;
        // page LSE over 16 tokens: 4 in this lane, the rest in the lanes 4 and 8
        // apart in this row (same page and slot, other token quarters)
        float sm = fast_exp2(dl[0]) + fast_exp2(dl[1]) + fast_exp2(dl[2]) + fast_exp2(dl[3]);
        sm += dpp<kRowRor4>(sm);
        sm += dpp<kRowRor8>(sm);
        float lse2;
        if (__any(!(sm >= 1e-30f && sm <= 1e30f))) {
          float mx = fmaxf(fmaxf(dl[0], dl[1]), fmaxf(dl[2], dl[3]));
          mx = fmaxf(mx, dpp<kRowRor4>(mx));
          mx = fmaxf(mx, dpp<kRowRor8>(mx));
          float s3 = fast_exp2(dl[0] - mx) + fast_exp2(dl[1] - mx) + fast_exp2(dl[2] - mx) +
                     fast_exp2(dl[3] - mx);
          s3 += dpp<kRowRor4>(s3);
          s3 += dpp<kRowRor8>(s3);
          lse2 = mx + fast_log2(s3);
        } else {
          lse2 = fast_log2(sm);
        }
        const float s2 = qmu2 + lse2;
        if (tok < 4 && jpg < n_fin) {
          outl[4 * sub + h][kWavePages * wv + 4 * k + row] = okp ? s2 * kLn2 : -INFINITY;
          if (okp) lse2_merge(pm[sub], ps[sub], s2, 1.f);
        }
      };
      sub_pass(0);
      if constexpr (NSUB > 1) sub_pass(1);
    }
  }

  // ---- this wave's (max, sum) of each head slot, for the page-mass
  // normalization: over the lanes 16 and 32 apart, by row swaps (lse2_merge
  // gives the same bits with its operands exchanged, so both lanes of a pair
  // agree) ----
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
    float ma, mb, sa, sb;
    float m = pm[sub], sm = ps[sub];
    swap16(m, ma, mb);
    swap16(sm, sa, sb);
    m = ma;
    sm = sa;
    lse2_merge(m, sm, mb, sb);
    swap32(m, ma, mb);
    swap32(sm, sa, sb);
    m = ma;
    sm = sa;
    lse2_merge(m, sm, mb, sb);
    if (lane < 4) red[wv][4 * sub + lane] = make_float2(m, sm);
  }
  __syncthreads();

  // ---- the workgroup's summarized pages: one 4-page piece per thread, each
  // head's kWgPages scores leave as one contiguous run ----
  constexpr int kPieces = kWgPages / 4;   // per head
  static_assert(kSlots * kPieces <= 64 * kScoreWaves, "one 4-page piece per thread");
  {
    const int t = threadIdx.x;
    const int p0 = kWgPages * g;
    const int nval = min(kWgPages, n_fin - p0);
    const int hh = t / kPieces, part = t % kPieces;
    float* dst = lse_out + (size_t)hh * p.max_pages + p0 + 4 * part;
    const bool vec = (p.max_pages & 3) == 0 && ((uintptr_t)p.page_lse & 15) == 0;
    if (hh < G && 4 * part < nval) {
      const float4 v = *reinterpret_cast<const float4*>(&outl[hh][4 * part]);
      if (vec && 4 * part + 4 <= nval) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        const float e[4] = {v.x, v.y, v.z, v.w};
        for (int i = 0; i < 4 && 4 * part + i < nval; ++i) dst[i] = e[i];
      }
    }
    // one (max, sum) partial per workgroup and head
    if (t < G && p.partials) {
      float pm2 = -INFINITY, ps2 = 0.f;
#pragma unroll
      for (int v2 = 0; v2 < kScoreWaves; ++v2) lse2_merge(pm2, ps2, red[v2][t].x, red[v2][t].y);
      p.partials[((size_t)b * p.hq + qhead0 + t) * W + g] = make_float2(pm2, ps2);
    }
  }
}

}  // namespace

ScorePlan plan_score(int32_t batch, int32_t hkv, int32_t max_pages) {
  // short-lived waves of about kScoreSteps steps each: many dispatch rounds
  // keep the end-of-launch tail small
  (void)batch;
  (void)hkv;
  ScorePlan pl;
  const long long steps = (long long)kScoreSteps * kScoreWaves;
  const long long nsteps = ((long long)max_pages + 3) / 4;
  pl.n_chunks = (int32_t)std::max(1LL, (nsteps + steps - 1) / steps);
  return pl;
}

hipError_t launch_score(int32_t rank, const uint16_t* q, const uint8_t* summ, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                        int32_t batch, int32_t hq, int32_t hkv, int32_t pending, float scale,
                        float* page_lse, float2* partials, const ScorePlan& plan,
                        hipStream_t stream) {
  const int32_t group = hq / hkv;
  ScoreParams p{q, summ, block_table, seq_lens, page_lse, partials, scale * kLog2e, num_blocks,
                max_pages, hq, hkv, plan.n_chunks, group, pending};
  dim3 grid(plan.n_chunks, hkv, batch);
  const dim3 blk(64 * kScoreWaves);
  const bool two = group > 4;   // two 4-head sub-passes
  switch (rank) {
    case 4:
      if (two) hipLaunchKernelGGL((score_kernel<4, 2>), grid, blk, 0, stream, p);
      else hipLaunchKernelGGL((score_kernel<4, 1>), grid, blk, 0, stream, p);
      break;
    case 8:
      if (two) hipLaunchKernelGGL((score_kernel<8, 2>), grid, blk, 0, stream, p);
      else hipLaunchKernelGGL((score_kernel<8, 1>), grid, blk, 0, stream, p);
      break;
    case 16:
      if (two) hipLaunchKernelGGL((score_kernel<16, 2>), grid, blk, 0, stream, p);
      else hipLaunchKernelGGL((score_kernel<16, 1>), grid, blk, 0, stream, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace locks
