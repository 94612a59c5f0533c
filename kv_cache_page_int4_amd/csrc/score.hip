// Page scoring from summaries: s_hat_j(q) = LSE_i((q.mu_j + (V_j^T q).c_i)/sqrt(d))
// (LOCKS explainer, technical summary sec. 2, reconstruction and selection).
//
// Work split.  A workgroup (one wave) owns a contiguous chunk of logical
// pages of one (sequence, KV head) and walks it in 16-page blocks, 4 pages
// per step; the records of the next step (and the block ids of the next
// block) are loaded while the current step computes.  Every record is read
// exactly once, with 16-byte loads.
//
// Per 4-page step one wave does:
//  * V^T q on the matrix cores: rows = (page, basis) pairs, K = head dim,
//    columns = the 4 query heads of the group repeated 4 times.  The int4
//    basis codes become bf16 values 136+n exactly (byte permute onto the
//    exponent of 128); the accumulator starts at -136*sum(q).  With the
//    rows ordered (page = lane/16, basis = register), lane l ends up holding
//    w[page l/16][k][head l%4] for all 8 k.
//  * the coefficient term on the vector units: lane l takes token l%16 of
//    page l/16 and pulls w[.][k][h] for the 4 heads from its own quad with DPP
//    broadcasts, so one int8->f32 conversion of c_ik serves all 4 heads.
//  * the page LSE over the 16 tokens of a page = one DPP row reduction.
// q.mu for a whole 16-page block is one more matrix-core product (int8
// centroid codes are exact in bf16), ordered so that each row of lanes finds
// its page's value in a register and its quad.
#include "locks_device.h"
#include "locks_internal.h"

namespace locks {

namespace {

constexpr uint32_t kMagic = 0x43434343u;  // bf16 high byte of 128.0

struct ScoreParams {
  const uint16_t* q;
  const uint8_t* summ;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* page_lse;
  float2* partials;
  int32_t num_blocks, max_pages, hq, hkv, n_chunks, pages_per_chunk;
};

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

struct StepLoads {
  uint4 va, vb;   // basis codes of (page tok/4, basis tok%4 and tok%4+4), dims 32*row..+32
  uint4 sv, sc;   // fp16 scales of page `row`
  uint2 cc;       // coefficient codes of token tok of page `row`
};

struct MuLoads {
  uint4 m0, m1;   // centroid codes of page pi(tok), dims 32*row..+32
  float smu[4];   // centroid scales of pages 4r + row
};

__global__ __launch_bounds__(64) void score_kernel(ScoreParams p) {
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int qhead0 = kvh * kG;
  const int row = lane >> 4;   // page slot of this lane in a 4-page step
  const int tok = lane & 15;   // token (coefficient lane) / MFMA row index

  int seq = p.seq_lens[b];
  seq = max(0, min(seq, p.max_pages * kB));
  const int n_fin = seq / kB;

  const uint8_t* __restrict__ summ_h = p.summ + (size_t)kvh * p.num_blocks * kRec;
  const int32_t* __restrict__ bt = p.block_table + (size_t)b * p.max_pages;
  float* __restrict__ lse_out = p.page_lse + ((size_t)b * p.hq + qhead0) * p.max_pages;

  const int jbeg = chunk * p.pages_per_chunk;
  const int jend = min(jbeg + p.pages_per_chunk, p.max_pages);
  const int jreal = min(jend, n_fin);
  const int n_blk = jreal > jbeg ? (jreal - jbeg + 15) / 16 : 0;

  // pages of this chunk past the covered blocks: not finalized
  for (int j = jbeg + 16 * n_blk + row; j < jend; j += 4)
    if (tok < 4) lse_out[(size_t)tok * p.max_pages + j] = -INFINITY;

  float pm = -INFINITY, ps = 0.f;   // running base-2 (max, sum) of head tok (tok < 4)
  if (n_blk > 0) {
    // q as MFMA B operands: column (lane%16) is head lane%4; K element
    // (step s, lane group g, e) is dim 32g + 8s + e.
    const int h = lane & 3;
    const uint16_t* qrow = p.q + ((size_t)b * p.hq + qhead0 + h) * kD + 32 * row;
    bf16x8 bq[4];
    float qsum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 8 * s);
      bq[s] = as_bf16x8(v);
      qsum += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
              bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
    }
    qsum += __shfl_xor(qsum, 16);
    qsum += __shfl_xor(qsum, 32);
    // the codes enter the product as 136 + n: start the accumulator at -136 sum(q)
    const float acc0_init = -136.f * qsum;
    const float c0 = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)

    // block ids of a 16-page block, one per lane (replicated in each row);
    // -1 marks a page that is not finalized or has an out-of-range block id
    auto load_bids = [&](int jb) -> int {
      const int j = jb + tok;
      const int v = bt[min(j, n_fin - 1)];
      return (j < n_fin && (unsigned)v < (unsigned)p.num_blocks) ? v : -1;
    };
    auto rec_of = [&](int bid) -> const uint8_t* {
      return summ_h + (size_t)(bid < 0 ? 0 : bid) * kRec;
    };
    auto issue_step = [&](int bids, int it) -> StepLoads {
      StepLoads L;
      const uint8_t* rv = rec_of(__shfl(bids, 4 * it + (tok >> 2))) + 64 * (lane & 3) + 16 * row;
      L.va = *reinterpret_cast<const uint4*>(rv);
      L.vb = *reinterpret_cast<const uint4*>(rv + 256);
      const uint8_t* rp = rec_of(__shfl(bids, 4 * it + row));
      L.sv = *reinterpret_cast<const uint4*>(rp + kOffSv);
      L.sc = *reinterpret_cast<const uint4*>(rp + kOffSc);
      L.cc = *reinterpret_cast<const uint2*>(rp + kOffC + 8 * tok);
      return L;
    };
    auto issue_mu = [&](int bids) -> MuLoads {
      MuLoads M;
      const int pm_ = 4 * (tok & 3) + (tok >> 2);
      const uint8_t* rm = rec_of(__shfl(bids, pm_)) + kOffMu + 32 * row;
      M.m0 = *reinterpret_cast<const uint4*>(rm);
      M.m1 = *reinterpret_cast<const uint4*>(rm + 16);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        M.smu[r] = half_lo(*reinterpret_cast<const uint16_t*>(rec_of(__shfl(bids, 4 * r + row)) + kOffSmu));
      return M;
    };

    int bids_cur = load_bids(jbeg);
    int bids_next = (n_blk > 1) ? load_bids(jbeg + 16) : -1;
    StepLoads nxt = issue_step(bids_cur, 0);
    MuLoads mu = issue_mu(bids_cur);

    for (int bk = 0; bk < n_blk; ++bk) {
      const int jb = jbeg + 16 * bk;
      // ---- q.mu for the 16 pages of this block (rows ordered page = 4r + g) ----
      float qmu[4];
      {
        f32x4 dm = {0.f, 0.f, 0.f, 0.f};
        dm = mfma16x16x32(i8x8_to_bf16(make_uint2(mu.m0.x, mu.m0.y)), bq[0], dm);
        dm = mfma16x16x32(i8x8_to_bf16(make_uint2(mu.m0.z, mu.m0.w)), bq[1], dm);
        dm = mfma16x16x32(i8x8_to_bf16(make_uint2(mu.m1.x, mu.m1.y)), bq[2], dm);
        dm = mfma16x16x32(i8x8_to_bf16(make_uint2(mu.m1.z, mu.m1.w)), bq[3], dm);
#pragma unroll
        for (int r = 0; r < 4; ++r) qmu[r] = dm[r] * mu.smu[r] * c0;
      }
      const int okrow_bids = bids_cur;
      float blk_lse[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const StepLoads cur = nxt;
        // prefetch the next step (next block's first step and centroids at it == 3)
        if (it < 3) {
          nxt = issue_step(bids_cur, it + 1);
        } else if (bk + 1 < n_blk) {
          nxt = issue_step(bids_next, 0);
          mu = issue_mu(bids_next);
        }
        const bool okp = __shfl(okrow_bids, 4 * it + row) >= 0;

        f32x4 acc0 = {acc0_init, acc0_init, acc0_init, acc0_init};
        f32x4 acc1 = acc0;
        acc0 = mfma16x16x32(nib8_to_bf16(cur.va.x), bq[0], acc0);
        acc1 = mfma16x16x32(nib8_to_bf16(cur.vb.x), bq[0], acc1);
        acc0 = mfma16x16x32(nib8_to_bf16(cur.va.y), bq[1], acc0);
        acc1 = mfma16x16x32(nib8_to_bf16(cur.vb.y), bq[1], acc1);
        acc0 = mfma16x16x32(nib8_to_bf16(cur.va.z), bq[2], acc0);
        acc1 = mfma16x16x32(nib8_to_bf16(cur.vb.z), bq[2], acc1);
        acc0 = mfma16x16x32(nib8_to_bf16(cur.va.w), bq[3], acc0);
        acc1 = mfma16x16x32(nib8_to_bf16(cur.vb.w), bq[3], acc1);

        // w[k] = (q.v_k) * s_V[k] * s_c[k] for head lane%4 (log2(e)/sqrt(d) applied later)
        const uint32_t svw[4] = {cur.sv.x, cur.sv.y, cur.sv.z, cur.sv.w};
        const uint32_t scw[4] = {cur.sc.x, cur.sc.y, cur.sc.z, cur.sc.w};
        float wk[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int k0 = r, k1 = r + 4;
          const float f0 = ((k0 & 1) ? half_hi(svw[k0 >> 1]) : half_lo(svw[k0 >> 1])) *
                           ((k0 & 1) ? half_hi(scw[k0 >> 1]) : half_lo(scw[k0 >> 1]));
          const float f1 = ((k1 & 1) ? half_hi(svw[k1 >> 1]) : half_lo(svw[k1 >> 1])) *
                           ((k1 & 1) ? half_hi(scw[k1 >> 1]) : half_lo(scw[k1 >> 1]));
          wk[k0] = acc0[r] * f0;
          wk[k1] = acc1[r] * f1;
        }
        float cf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cf[e] = (float)(int8_t)(cur.cc.x >> (8 * e));
          cf[4 + e] = (float)(int8_t)(cur.cc.y >> (8 * e));
        }
        // deviation logits (without q.mu) of token `tok`, 4 heads, base 2
        float dl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          dl[0] = fmaf(quad_bcast<0>(wk[k]), cf[k], dl[0]);
          dl[1] = fmaf(quad_bcast<1>(wk[k]), cf[k], dl[1]);
          dl[2] = fmaf(quad_bcast<2>(wk[k]), cf[k], dl[2]);
          dl[3] = fmaf(quad_bcast<3>(wk[k]), cf[k], dl[3]);
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) dl[hh] *= c0;
        // page LSE over the 16 tokens: no shift unless a sum leaves the safe range
        float sm[4];
        bool bad = false;
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          sm[hh] = row_sum16(fast_exp2(dl[hh]));
          bad |= !(sm[hh] >= 1e-30f && sm[hh] <= 1e30f);
        }
        float lse2[4];
        if (__any(bad)) {
#pragma unroll
          for (int hh = 0; hh < 4; ++hh) {
            const float mx = row_max16(dl[hh]);
            lse2[hh] = mx + fast_log2(row_sum16(fast_exp2(dl[hh] - mx)));
          }
        } else {
#pragma unroll
          for (int hh = 0; hh < 4; ++hh) lse2[hh] = fast_log2(sm[hh]);
        }
        const float qm0 = quad_bcast<0>(qmu[it]), qm1 = quad_bcast<1>(qmu[it]);
        const float qm2 = quad_bcast<2>(qmu[it]), qm3 = quad_bcast<3>(qmu[it]);
        const float s2 = (tok == 0) ? qm0 + lse2[0] : (tok == 1) ? qm1 + lse2[1]
                       : (tok == 2) ? qm2 + lse2[2] : qm3 + lse2[3];
        blk_lse[it] = okp ? s2 * kLn2 : -INFINITY;
        if (tok < 4 && okp) lse2_merge(pm, ps, s2, 1.f);
      }
      // one coalesced store per block: lane 16h + i takes page jb + i of head
      // h, computed at step i/4 by lane 16*(i%4) + h
      {
        const int hh = lane >> 4, i = lane & 15;
        const int src = 16 * (i & 3) + hh;
        const float v0 = __shfl(blk_lse[0], src), v1 = __shfl(blk_lse[1], src);
        const float v2 = __shfl(blk_lse[2], src), v3 = __shfl(blk_lse[3], src);
        const int st = i >> 2;
        const float v = (st == 0) ? v0 : (st == 1) ? v1 : (st == 2) ? v2 : v3;
        const int j = jb + i;
        if (j < jend) lse_out[(size_t)hh * p.max_pages + j] = v;
      }
      if (bk + 1 < n_blk) {
        bids_cur = bids_next;
        bids_next = (bk + 2 < n_blk) ? load_bids(jb + 32) : -1;
      }
    }
  }

  // ---- per-chunk (max, sum) of each head, for the page-mass normalization ----
  float m2 = __shfl_xor(pm, 16), s2 = __shfl_xor(ps, 16);
  lse2_merge(pm, ps, m2, s2);
  m2 = __shfl_xor(pm, 32);
  s2 = __shfl_xor(ps, 32);
  lse2_merge(pm, ps, m2, s2);
  if (lane < 4 && p.partials)
    p.partials[((size_t)b * p.hq + qhead0 + lane) * p.n_chunks + chunk] = make_float2(pm, ps);
}

}  // namespace

ScorePlan plan_score(int32_t batch, int32_t hkv, int32_t max_pages) {
  // one wave per workgroup; aim for >= ~8k workgroups at long context
  ScorePlan pl;
  int bpw = 1;
  const long long groups = (long long)batch * hkv;
  while (bpw < 8) {
    const long long chunk = 16LL * bpw * 2;
    if (groups * ((max_pages + chunk - 1) / chunk) < 8192) break;
    bpw *= 2;
  }
  pl.blocks16_per_wave = bpw;
  pl.pages_per_chunk = 16 * bpw;
  pl.n_chunks = (max_pages + pl.pages_per_chunk - 1) / pl.pages_per_chunk;
  return pl;
}

hipError_t launch_score(const uint16_t* q, const uint8_t* summ, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                        int32_t batch, int32_t hq, int32_t hkv, float* page_lse,
                        float2* partials, const ScorePlan& plan, hipStream_t stream) {
  ScoreParams p{q, summ, block_table, seq_lens, page_lse, partials, num_blocks, max_pages, hq,
                hkv, plan.n_chunks, plan.pages_per_chunk};
  dim3 grid(plan.n_chunks, hkv, batch);
  hipLaunchKernelGGL(score_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
