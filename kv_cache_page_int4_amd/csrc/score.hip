// Page scoring from summaries: s_hat_j(q) = LSE_i((q.mu_j + (V_j^T q).c_i)/sqrt(d))
// (LOCKS explainer, technical summary sec. 2, reconstruction and selection).
//
// Work split.  A workgroup (4 waves) owns a contiguous chunk of logical pages
// of one (sequence, KV head); each wave walks 16-page blocks, 4 pages per
// step.  Every record is read exactly once, with 16-byte loads.
//
// Per 4-page step one wave does:
//  * V^T q on the matrix cores: rows = (page, basis) pairs, K = head dim,
//    columns = the 4 query heads of the group repeated 4 times.  The int4
//    basis codes become bf16 values 136+n exactly (byte permute onto the
//    exponent of 128); the 136*sum(q) offset is removed afterwards.  With the
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

constexpr int kWaves = 4;
constexpr uint32_t kMagic = 0x43434343u;  // bf16 high byte of 128.0

struct ScoreParams {
  const uint16_t* q;
  const uint8_t* summ;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* page_lse;
  float2* partials;
  int32_t num_blocks, max_pages, hq, hkv, n_chunks, blocks16_per_wave;
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

__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int qhead0 = kvh * kG;
  const int row = lane >> 4;   // page slot of this lane in a 4-page step
  const int tok = lane & 15;   // token (coefficient lane) / MFMA row index

  int seq = p.seq_lens[b];
  seq = max(0, min(seq, p.max_pages * kB));
  const int n_fin = seq / kB;

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
  const float bias = 136.f * qsum;               // sum_d q_d * (136 + n_d) - sum_d q_d n_d
  const float c0 = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)

  const uint8_t* summ_h = p.summ + (size_t)kvh * p.num_blocks * kRec;
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
  float* lse_out = p.page_lse + ((size_t)b * p.hq + qhead0) * p.max_pages;

  // running base-2 (max, sum) of this lane's head (lanes with tok < 4)
  float pm = -INFINITY, ps = 0.f;

  const int chunk_pages = kWaves * p.blocks16_per_wave * 16;
  for (int blk = 0; blk < p.blocks16_per_wave; ++blk) {
    const int jb = chunk * chunk_pages + (wave * p.blocks16_per_wave + blk) * 16;
    if (jb >= p.max_pages) break;
    if (jb >= n_fin) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int j = jb + 4 * it + row;
        if (tok < 4 && j < p.max_pages) lse_out[(size_t)tok * p.max_pages + j] = -INFINITY;
      }
      continue;
    }
    auto page_rec = [&](int j, bool& ok) -> const uint8_t* {
      const int jj = min(j, n_fin - 1);
      int bid = bt[jj];
      ok = (j < n_fin) && ((unsigned)bid < (unsigned)p.num_blocks);
      bid = ((unsigned)bid < (unsigned)p.num_blocks) ? bid : 0;
      return summ_h + (size_t)bid * kRec;
    };

    // ---- q.mu for the 16 pages of this block (rows ordered page = 4r + g) ----
    float qmu[4];
    {
      const int rho = tok;
      const int pm_ = 4 * (rho & 3) + (rho >> 2);
      bool ok;
      const uint8_t* rm = page_rec(jb + pm_, ok) + kOffMu + 32 * row;
      const uint4 m0 = *reinterpret_cast<const uint4*>(rm);
      const uint4 m1 = *reinterpret_cast<const uint4*>(rm + 16);
      f32x4 dm = {0.f, 0.f, 0.f, 0.f};
      dm = mfma16x16x32(i8x8_to_bf16(make_uint2(m0.x, m0.y)), bq[0], dm);
      dm = mfma16x16x32(i8x8_to_bf16(make_uint2(m0.z, m0.w)), bq[1], dm);
      dm = mfma16x16x32(i8x8_to_bf16(make_uint2(m1.x, m1.y)), bq[2], dm);
      dm = mfma16x16x32(i8x8_to_bf16(make_uint2(m1.z, m1.w)), bq[3], dm);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok2;
        const uint8_t* rs = page_rec(jb + 4 * r + row, ok2);
        const float smu = half_lo(*reinterpret_cast<const uint16_t*>(rs + kOffSmu));
        qmu[r] = dm[r] * smu * c0;
      }
    }

#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int j0 = jb + 4 * it;
      // ---- basis rows: lane -> (page tok/4, basis tok%4 [+4], dim chunk row) ----
      bool okv;
      const uint8_t* rv = page_rec(j0 + (tok >> 2), okv) + 64 * (lane & 3) + 16 * row;
      const uint4 va = *reinterpret_cast<const uint4*>(rv);
      const uint4 vb = *reinterpret_cast<const uint4*>(rv + 256);
      // ---- scales and coefficients of page `row` ----
      bool okp;
      const uint8_t* rp = page_rec(j0 + row, okp);
      const uint4 sv = *reinterpret_cast<const uint4*>(rp + kOffSv);
      const uint4 sc = *reinterpret_cast<const uint4*>(rp + kOffSc);
      const uint2 cc = *reinterpret_cast<const uint2*>(rp + kOffC + 8 * tok);

      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      acc0 = mfma16x16x32(nib8_to_bf16(va.x), bq[0], acc0);
      acc1 = mfma16x16x32(nib8_to_bf16(vb.x), bq[0], acc1);
      acc0 = mfma16x16x32(nib8_to_bf16(va.y), bq[1], acc0);
      acc1 = mfma16x16x32(nib8_to_bf16(vb.y), bq[1], acc1);
      acc0 = mfma16x16x32(nib8_to_bf16(va.z), bq[2], acc0);
      acc1 = mfma16x16x32(nib8_to_bf16(vb.z), bq[2], acc1);
      acc0 = mfma16x16x32(nib8_to_bf16(va.w), bq[3], acc0);
      acc1 = mfma16x16x32(nib8_to_bf16(vb.w), bq[3], acc1);

      // w'[k] = (q.v_k) * s_V[k] * s_c[k] * log2(e)/sqrt(d) for head lane%4
      const uint32_t svw[4] = {sv.x, sv.y, sv.z, sv.w};
      const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
      float wk[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k0 = r, k1 = r + 4;
        const float f0 = ((k0 & 1) ? half_hi(svw[k0 >> 1]) : half_lo(svw[k0 >> 1])) *
                         ((k0 & 1) ? half_hi(scw[k0 >> 1]) : half_lo(scw[k0 >> 1]));
        const float f1 = ((k1 & 1) ? half_hi(svw[k1 >> 1]) : half_lo(svw[k1 >> 1])) *
                         ((k1 & 1) ? half_hi(scw[k1 >> 1]) : half_lo(scw[k1 >> 1]));
        wk[k0] = (acc0[r] - bias) * (f0 * c0);
        wk[k1] = (acc1[r] - bias) * (f1 * c0);
      }
      float cf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cf[e] = (float)(int8_t)(cc.x >> (8 * e));
        cf[4 + e] = (float)(int8_t)(cc.y >> (8 * e));
      }
      // deviation logits (base 2, without q.mu) of token `tok`, 4 heads
      float dl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        dl[0] = fmaf(quad_bcast<0>(wk[k]), cf[k], dl[0]);
        dl[1] = fmaf(quad_bcast<1>(wk[k]), cf[k], dl[1]);
        dl[2] = fmaf(quad_bcast<2>(wk[k]), cf[k], dl[2]);
        dl[3] = fmaf(quad_bcast<3>(wk[k]), cf[k], dl[3]);
      }
      float lse2[4];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float mx = row_max16(dl[hh]);
        const float sm = row_sum16(fast_exp2(dl[hh] - mx));
        lse2[hh] = mx + fast_log2(sm);
      }
      const float qm0 = quad_bcast<0>(qmu[it]), qm1 = quad_bcast<1>(qmu[it]);
      const float qm2 = quad_bcast<2>(qmu[it]), qm3 = quad_bcast<3>(qmu[it]);
      float s2 = (tok == 0) ? qm0 + lse2[0] : (tok == 1) ? qm1 + lse2[1]
               : (tok == 2) ? qm2 + lse2[2] : qm3 + lse2[3];
      const int j = j0 + row;
      if (tok < 4) {
        if (j < p.max_pages) lse_out[(size_t)tok * p.max_pages + j] = okp ? s2 * kLn2 : -INFINITY;
        if (okp) lse2_merge(pm, ps, s2, 1.f);
      }
    }
  }

  // ---- per-chunk (max, sum) of each head, for the page-mass normalization ----
  __shared__ float2 red[kWaves][4];
  {
    float m2 = __shfl_xor(pm, 16), s2 = __shfl_xor(ps, 16);
    lse2_merge(pm, ps, m2, s2);
    m2 = __shfl_xor(pm, 32);
    s2 = __shfl_xor(ps, 32);
    lse2_merge(pm, ps, m2, s2);
    if (lane < 4) red[wave][lane] = make_float2(pm, ps);
  }
  __syncthreads();
  if (threadIdx.x < 4 && p.partials) {
    float m = red[0][threadIdx.x].x, s = red[0][threadIdx.x].y;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) lse2_merge(m, s, red[w][threadIdx.x].x, red[w][threadIdx.x].y);
    p.partials[((size_t)b * p.hq + qhead0 + threadIdx.x) * p.n_chunks + chunk] = make_float2(m, s);
  }
}

}  // namespace

ScorePlan plan_score(int32_t batch, int32_t hkv, int32_t max_pages) {
  ScorePlan pl;
  int bpw = 1;
  const long long groups = (long long)batch * hkv;
  while (bpw < 8) {
    const long long chunk = (long long)kWaves * 16 * bpw * 2;
    if (groups * ((max_pages + chunk - 1) / chunk) < 2048) break;
    bpw *= 2;
  }
  pl.blocks16_per_wave = bpw;
  pl.pages_per_chunk = kWaves * 16 * bpw;
  pl.n_chunks = (max_pages + pl.pages_per_chunk - 1) / pl.pages_per_chunk;
  return pl;
}

hipError_t launch_score(const uint16_t* q, const uint8_t* summ, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                        int32_t batch, int32_t hq, int32_t hkv, float* page_lse,
                        float2* partials, const ScorePlan& plan, hipStream_t stream) {
  ScoreParams p{q, summ, block_table, seq_lens, page_lse, partials, num_blocks, max_pages, hq,
                hkv, plan.n_chunks, plan.blocks16_per_wave};
  dim3 grid(plan.n_chunks, hkv, batch);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace locks
