// Page-summary builder: runs when a page is finalized, off the decode path
// (LOCKS explainer, technical summary sec. 2, core mechanism: the centroid,
// a small eigendecomposition of the page's centered keys, the top-r
// eigenvectors and one coefficient vector per token; int4 basis, int8
// coefficients and centroid).
//
// One wave per (page, KV head):
//  1. load the 16x128 bf16 keys, centroid mu by DPP row sums, X = K - mu in fp32;
//  2. Gram matrix X X^T (16x16) on the matrix cores (fp32 16x16x4);
//  3. cyclic Jacobi on the Gram matrix in LDS: pairs (i, i^m) for m = 1..15
//     form 8 disjoint rotations per step; each lane owns one 2x2 block of the
//     matrix and one row-pair of the eigenvector matrix; sweeps stop once the
//     off-diagonal mass is below 1e-12 of the total (at most 10);
//  4. the top-8 eigenpairs (descending, ties to the lower index) give the
//     basis v_k = X^T u_k normalized to unit length (the dual of the d x d
//     scatter's eigenproblem), zeroed when lambda_k <= 1e-5 lambda_1 or when
//     the page is constant to rounding;
//  5. sign: the largest-|entry| component of v_k is made positive (lowest dim
//     on ties); coefficients c_i = V^T x_i are projections on the unquantized
//     basis;
//  6. symmetric quantization with fp16 scales (max|x|/7 for the basis,
//     max|x|/127 for coefficients and centroid, round half to even) and
//     packing into the 832-byte record.
// With a given basis (the shared-basis selector the pages contrast LOCKS
// with), steps 2-5 are replaced by that basis: the record keeps the page's own
// centroid and coefficients c_i = V^T x_i in the given basis.
#include "locks_device.h"
#include "locks_internal.h"

namespace locks {

namespace {

constexpr int kSweeps = 10;
constexpr float kTau = 1e-5f;
constexpr float kEpsConst = 1e-12f;

typedef float f32x4v __attribute__((ext_vector_type(4)));

// whole-wave sum and max on DPP and the row swaps (no LDS round trips)
__device__ __forceinline__ float wave_sum(float x) { return wave_sum_f(x); }
__device__ __forceinline__ float wave_max(float x) { return wave_max_f(x); }

// fp16 scale of a max-magnitude: round to nearest even, saturate at 65504.
__device__ __forceinline__ float fp16_scale(float m, float qmax) {
  float s = m / qmax;
  s = fminf(s, 65504.f);
  return (float)(_Float16)s;
}
__device__ __forceinline__ uint32_t fp16_bits(float s) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s);
}
__device__ __forceinline__ int quant(float x, float s, int qmax) {
  if (!(s > 0.f)) return 0;
  float v = rintf(x / s);
  v = fminf(fmaxf(v, (float)-qmax), (float)qmax);
  return (int)v;
}

// Rotation (c, s) that zeroes G[p][q] of the 2x2 block [[app, apq], [apq, aqq]]
// (classical symmetric Schur decomposition: t = tan of the angle =
// sign(tau) w / (|tau| + sqrt(tau^2 + w^2)) with tau = aqq - app, w = 2 apq,
// c = 1 / sqrt(1 + t^2), s = t c), branch-free, with the hardware's
// reciprocal, square root and reciprocal square root (about 1 ulp each): any
// rotation near the zeroing one serves Jacobi, which goes on until the
// off-diagonal mass is negligible, and c^2 + s^2 = 1 holds to a few ulp.
__device__ __forceinline__ void jacobi_rot(float app, float apq, float aqq, float& c, float& s) {
  const bool skip = !(fabsf(apq) > 1e-30f * (fabsf(app) + fabsf(aqq)));   // also apq == 0
  const float tau = aqq - app, w = 2.f * apq;
  const float t = (tau < 0.f ? -w : w) *
                  __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, w * w)));
  const float cc = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f));
  c = skip ? 1.f : cc;
  s = skip ? 0.f : t * cc;
}

// Record of rank R (R = 4, 8, 16): the rank-8 layout with every field sized
// by R, in 32-bit words: basis codes [0, 16R), coefficient codes
// [16R, 20R), centroid codes [20R, 20R + 32), s_V [20R + 32, +R/2), s_c the
// next R/2 words, s_mu the low half of the word after, zero up to the record
// size (the fields' 84R + 130 bytes rounded up to 64).
template <int R>
struct RecLayout {
  static constexpr int kBytes = rec_bytes(R);
  static constexpr int kWC = 16 * R, kWMu = 20 * R, kWSv = 20 * R + 32;
  static constexpr int kWSc = kWSv + R / 2, kWSmu = kWSc + R / 2;
};

// LDS of one build (one wave).  The keys are not kept: the basis and the
// coefficients read the page-head's 4 KB again (from L2, where the first
// read left it) and centre it again (k - mu in fp32, the same values the
// centring step computes).  The eigen-solver's matrices are dead once the
// basis is formed, and the packing buffers and the coefficients take their
// place.  7 KB at rank 8: the registers, not the LDS, bound the builds per CU.
template <int R>
struct BuildSmem {
  union {
    struct {
      float G[kB][kB + 1];     // Gram matrix -> eigenvalues on the diagonal
      float U[kB][kB + 1];     // eigenvectors (columns)
      float cs[8][2] __attribute__((aligned(16)));   // rotations of the current step
    } e;                       // eigen-solver, until the basis is formed
    struct {
      int8_t vq[R][kD];
      uint32_t rec[RecLayout<R>::kBytes / 4];
      float C[kB][R];          // unquantized coefficients
    } q;                       // coefficients, quantization and packing, after it
  } u;
  float V[R][kD + 4];      // unquantized basis, [k][d]
  float mu[kD] __attribute__((aligned(16)));
  int order[kB];
};

// Which block a workgroup summarizes: entry blockIdx.x of a list, or (for
// incremental finalization) the last full page of sequence blockIdx.x when
// that sequence's length is a positive multiple of the page size -- the page
// that the newest token just completed.
struct BlockSource {
  const int32_t* block_ids;    // list mode
  const int32_t* seq_lens;     // finalize mode: [batch]
  const int32_t* block_table;  // finalize mode: [batch][max_pages]
  int32_t max_pages;
  bool from_seq;
  int64_t k_layer_stride;      // finalize mode: layer blockIdx.z of the caches
  int64_t summ_layer_stride;
};

template <int R>
__global__ __launch_bounds__(64) void build_kernel(const uint16_t* __restrict__ kc, int64_t bs,
                                                   int64_t hs, int64_t ts, BlockSource src,
                                                   int32_t n_blocks, int32_t num_blocks,
                                                   int32_t hkv, uint8_t* __restrict__ summ,
                                                   float* __restrict__ raw,
                                                   const float* __restrict__ basis) {
  using RL = RecLayout<R>;
  __shared__ BuildSmem<R> sm;
  const int lane = threadIdx.x;
  const int bi = blockIdx.x, kvh = blockIdx.y;
  kc += (size_t)blockIdx.z * src.k_layer_stride;
  summ += (size_t)blockIdx.z * src.summ_layer_stride;
  int blk;
  if (src.from_seq) {
    const int seq = src.seq_lens[bi];
    const int j = seq / kB - 1;
    blk = (seq > 0 && seq % kB == 0 && j < src.max_pages)
              ? src.block_table[(size_t)bi * src.max_pages + j] : -1;
  } else {
    blk = src.block_ids[bi];
  }
  if ((unsigned)blk >= (unsigned)num_blocks) return;   // whole workgroup, uniform
  const int t = lane & 15, g = lane >> 4;

  // ---- 1. keys, centroid, deviations ----
  const uint16_t* kp = kc + (size_t)blk * bs + (size_t)kvh * hs + (size_t)t * ts + 32 * g;
  float x[32];
  float ksq = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 v = *reinterpret_cast<const uint4*>(kp + 8 * s);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * s + 2 * e] = bf16_lo(w[e]);
      x[8 * s + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    ksq = fmaf(x[e], x[e], ksq);
    const float m = row_sum16(x[e]) * (1.f / 16.f);
    x[e] -= m;
    if (t == 0) sm.mu[32 * g + e] = m;
  }
  ksq = wave_sum(ksq);

  const int d0 = 2 * lane;   // basis dims owned by this lane: d0, d0 + 1
  // this page-head's keys, read again below: token tt, dims d .. d + 1
  const uint16_t* kpage = kc + (size_t)blk * bs + (size_t)kvh * hs;
  auto key_pair = [&](int tt, int d) {
    return *reinterpret_cast<const uint32_t*>(kpage + (size_t)tt * ts + d);
  };
  if (basis) {
    const float* bk = basis + (size_t)kvh * R * kD;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      sm.V[k][d0] = bk[k * kD + d0];
      sm.V[k][d0 + 1] = bk[k * kD + d0 + 1];
    }
    __syncthreads();
  } else {
    // ---- 2. Gram matrix on the matrix cores: K index (step s, group g) = dim 32g+s ----
    f32x4v gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 32; ++s) gacc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], x[s], gacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u.e.G[4 * g + r][t] = gacc[r];
    for (int i = lane; i < kB * kB; i += 64) sm.u.e.U[i >> 4][i & 15] = ((i >> 4) == (i & 15)) ? 1.f : 0.f;
    __syncthreads();
    // symmetrize (the product is symmetric up to rounding order)
    for (int i = lane; i < kB * kB; i += 64) {
      const int a = i >> 4, b = i & 15;
      if (a < b) {
        const float v = 0.5f * (sm.u.e.G[a][b] + sm.u.e.G[b][a]);
        sm.u.e.G[a][b] = v;
        sm.u.e.G[b][a] = v;
      }
    }
    __syncthreads();

    // ---- 3. cyclic Jacobi ----
    // A step m (1..15) rotates the 8 disjoint index pairs (i, i ^ m).  Lane
    // (ia, ib) owns the 2x2 block of G at row pair ia and column pair ib
    // (read from and written back to LDS); the diagonal lanes compute their
    // pair's rotation and publish (c, s) in LDS.  The eigenvector matrix stays
    // in registers: lane l holds row l % 16 of U and turns it by all 8
    // rotations of the step, whose column indices are constants once the
    // steps are unrolled.  The workgroup is one wave (launch bound 64).
    const int ia = lane >> 3, ib = lane & 7;   // row pair, column pair of this lane's block
    const int urow = lane & 15;
    float u[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) u[j] = (j == urow) ? 1.f : 0.f;
    for (int sweep = 0; sweep < kSweeps; ++sweep) {
      // this lane's pair indices, opaque to the compiler: the block addresses
      // of the 15 steps are recomputed in every sweep instead of being held
      // in registers across the sweeps
      int iav = ia, ibv = ib;
      asm volatile("" : "+v"(iav), "+v"(ibv));
#pragma unroll
      for (int m = 1; m < 16; ++m) {
        const int hb = 31 - __builtin_clz(m);
        auto pair_p = [&](int pi) { return ((pi >> hb) << (hb + 1)) | (pi & ((1 << hb) - 1)); };
        const int a0 = pair_p(iav), a1 = a0 ^ m, b0 = pair_p(ibv), b1 = b0 ^ m;
        const float g00 = sm.u.e.G[a0][b0], g01 = sm.u.e.G[a0][b1], g10 = sm.u.e.G[a1][b0], g11 = sm.u.e.G[a1][b1];
        {
          // every lane computes (branch-free); the diagonal lanes publish
          float c, s;
          jacobi_rot(g00, 0.5f * (g01 + g10), g11, c, s);
          if (ia == ib) *reinterpret_cast<float2*>(sm.u.e.cs[ia]) = make_float2(c, s);
        }
        // one wave: its LDS accesses complete in program order, so the reads
        // below see the rotations just written; only the compiler is kept
        // from reordering them.  All of the step's rotations are read at once.
        asm volatile("" ::: "memory");
        const float2 csa = *reinterpret_cast<const float2*>(sm.u.e.cs[ia]);
        const float2 csb = *reinterpret_cast<const float2*>(sm.u.e.cs[ib]);
        float4 cs4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cs4[i] = *reinterpret_cast<const float4*>(&sm.u.e.cs[2 * i][0]);
        const float ca = csa.x, sa = csa.y, cb = csb.x, sb = csb.y;
        // T = G J (columns b0, b1), then G' = J^T T (rows a0, a1)
        const float t00 = g00 * cb - g01 * sb, t01 = g00 * sb + g01 * cb;
        const float t10 = g10 * cb - g11 * sb, t11 = g10 * sb + g11 * cb;
        float n00 = ca * t00 - sa * t10, n01 = ca * t01 - sa * t11;
        float n10 = sa * t00 + ca * t10, n11 = sa * t01 + ca * t11;
        if (ia == ib) {
          n01 = 0.f;
          n10 = 0.f;
        }
        sm.u.e.G[a0][b0] = n00;
        sm.u.e.G[a0][b1] = n01;
        sm.u.e.G[a1][b0] = n10;
        sm.u.e.G[a1][b1] = n11;
        // U' = U J on this lane's row: all 8 rotations
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float c = (k & 1) ? cs4[k >> 1].z : cs4[k >> 1].x;
          const float s = (k & 1) ? cs4[k >> 1].w : cs4[k >> 1].y;
          const int p0 = pair_p(k), p1 = p0 ^ m;
          const float up = u[p0], uq = u[p1];
          u[p0] = c * up - s * uq;
          u[p1] = s * up + c * uq;
        }
        // apply the rotations now: left free, the compiler sinks them to the
        // end of the sweep and holds all 120 rotations in registers
        asm volatile("" : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]),
                     "+v"(u[5]), "+v"(u[6]), "+v"(u[7]), "+v"(u[8]), "+v"(u[9]), "+v"(u[10]),
                     "+v"(u[11]), "+v"(u[12]), "+v"(u[13]), "+v"(u[14]), "+v"(u[15])
                     :: "memory");
      }
      // converged when the off-diagonal mass is below 1e-12 of the total
      // (off-norm 1e-6 relative: far below what the codes and fp16 scales resolve)
      float off = 0.f, tot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * lane + e, a = i >> 4, b = i & 15;
        const float v = sm.u.e.G[a][b];
        tot = fmaf(v, v, tot);
        if (a != b) off = fmaf(v, v, off);
      }
      off = wave_sum(off);
      tot = wave_sum(tot);
      if (!(off > 1e-12f * tot)) break;
    }
    if (lane < kB) {
#pragma unroll
      for (int j = 0; j < kB; ++j) sm.u.e.U[urow][j] = u[j];
    }

    // ---- 4. order eigenpairs: descending eigenvalue, ties to the lower index ----
    if (lane < 16) {
      const float lj = sm.u.e.G[lane][lane];
      int rank = 0;
      for (int i = 0; i < 16; ++i) {
        const float li = sm.u.e.G[i][i];
        rank += (li > lj) || (li == lj && i < lane);
      }
      sm.order[rank] = lane;
    }
    __syncthreads();
    const float lam1 = sm.u.e.G[sm.order[0]][sm.order[0]];
    const bool page_has_basis = lam1 > kEpsConst * ksq;

    // basis v_k = X^T u_k / |X^T u_k|; lane owns dims 2*lane, 2*lane+1
    const float mu0 = sm.mu[d0], mu1 = sm.mu[d0 + 1];
    float2 xr[kB];
#pragma unroll
    for (int tt = 0; tt < kB; ++tt) {
      const uint32_t kw = key_pair(tt, d0);
      xr[tt] = make_float2(bf16_lo(kw) - mu0, bf16_hi(kw) - mu1);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = sm.order[k];
      const float lk = sm.u.e.G[j][j];
      const bool keep = page_has_basis && (lk > kTau * lam1);
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int tt = 0; tt < kB; ++tt) {
        const float uu = sm.u.e.U[tt][j];
        v0 = fmaf(xr[tt].x, uu, v0);
        v1 = fmaf(xr[tt].y, uu, v1);
      }
      const float nrm2 = wave_sum(fmaf(v1, v1, v0 * v0));
      const float inv = (keep && nrm2 > 0.f) ? 1.f / sqrtf(nrm2) : 0.f;
      v0 *= inv;
      v1 *= inv;
      // sign: the largest |v| (lowest dim on ties) is made positive
      const float a0v = fabsf(v0), a1v = fabsf(v1);
      const float amax = wave_max(fmaxf(a0v, a1v));
      const uint32_t cand = (a0v == amax) ? (uint32_t)d0 : (a1v == amax) ? (uint32_t)(d0 + 1) : 0xFFFFu;
      const int bidx = __builtin_amdgcn_readfirstlane((int)wave_min_u(cand));
      const float mine = (bidx & 1) ? v1 : v0;
      const float bval = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), bidx >> 1));
      if (bval < 0.f) {
        v0 = -v0;
        v1 = -v1;
      }
      sm.V[k][d0] = v0;
      sm.V[k][d0 + 1] = v1;
    }
    __syncthreads();
  }

  // coefficients c_ik = v_k . x_i : lane -> token t, columns
  // (R/4)*(lane>>4) .. +R/4
  {
    constexpr int kPer = R / 4;
    const int tk = lane & 15, k0 = kPer * (lane >> 4);
    float cc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) cc[j] = 0.f;
    for (int d = 0; d < kD; d += 2) {
      const uint32_t kw = key_pair(tk, d);
      const float2 m = *reinterpret_cast<const float2*>(&sm.mu[d]);
      const float xa = bf16_lo(kw) - m.x, xb = bf16_hi(kw) - m.y;
#pragma unroll
      for (int j = 0; j < kPer; ++j) cc[j] = fmaf(xa, sm.V[k0 + j][d], cc[j]);
#pragma unroll
      for (int j = 0; j < kPer; ++j) cc[j] = fmaf(xb, sm.V[k0 + j][d + 1], cc[j]);
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) sm.u.q.C[tk][k0 + j] = cc[j];
  }
  __syncthreads();

  // ---- 6. quantize + pack ----
  // centroid
  const float mu0 = sm.mu[d0], mu1 = sm.mu[d0 + 1];
  const float s_mu = fp16_scale(wave_max(fmaxf(fabsf(mu0), fabsf(mu1))), 127.f);
  const int mq0 = quant(mu0, s_mu, 127), mq1 = quant(mu1, s_mu, 127);
  // basis scales and codes
  float s_v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float a = sm.V[k][d0], b2 = sm.V[k][d0 + 1];
    s_v[k] = fp16_scale(wave_max(fmaxf(fabsf(a), fabsf(b2))), 7.f);
    sm.u.q.vq[k][d0] = (int8_t)quant(a, s_v[k], 7);
    sm.u.q.vq[k][d0 + 1] = (int8_t)quant(b2, s_v[k], 7);
  }
  // coefficient scales: column k max over the 16 tokens
  float s_c[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float a = (lane < 16) ? fabsf(sm.u.q.C[lane][k]) : 0.f;
    s_c[k] = fp16_scale(wave_max(a), 127.f);
  }
  __syncthreads();
  // record words: basis, coefficients, centroid, s_V, s_c, s_mu, zero
  uint8_t* mub = reinterpret_cast<uint8_t*>(&sm.u.q.rec[RL::kWMu]);
  mub[d0] = (uint8_t)(int8_t)mq0;
  mub[d0 + 1] = (uint8_t)(int8_t)mq1;
  for (int wi = lane; wi < 16 * R; wi += 64) {
    const int k = wi >> 4, w = wi & 15;
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = (uint32_t)sm.u.q.vq[k][8 * w + m] & 0xFu;
      const uint32_t hi = (uint32_t)sm.u.q.vq[k][8 * w + 4 + m] & 0xFu;
      word |= (lo | (hi << 4)) << (8 * m);
    }
    sm.u.q.rec[wi] = word;
  }
  // coefficient words: token tk holds R/4 words of 4 codes each
  if (lane < 4 * R) {
    constexpr int kWpt = R / 4;
    const int tk = lane / kWpt, kh = 4 * (lane % kWpt);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sce = s_c[0];
#pragma unroll
      for (int k = 1; k < R; ++k) sce = (k == kh + e) ? s_c[k] : sce;
      word |= ((uint32_t)(uint8_t)(int8_t)quant(sm.u.q.C[tk][kh + e], sce, 127)) << (8 * e);
    }
    sm.u.q.rec[RL::kWC + lane] = word;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      sm.u.q.rec[RL::kWSv + i] = fp16_bits(s_v[2 * i]) | (fp16_bits(s_v[2 * i + 1]) << 16);
      sm.u.q.rec[RL::kWSc + i] = fp16_bits(s_c[2 * i]) | (fp16_bits(s_c[2 * i + 1]) << 16);
    }
    sm.u.q.rec[RL::kWSmu] = fp16_bits(s_mu);
    for (int i = RL::kWSmu + 1; i < RL::kBytes / 4; ++i) sm.u.q.rec[i] = 0u;
  }
  __syncthreads();
  uint32_t* dst =
      reinterpret_cast<uint32_t*>(summ + ((size_t)kvh * num_blocks + blk) * RL::kBytes);
  for (int wi = lane; wi < RL::kBytes / 4; wi += 64) dst[wi] = sm.u.q.rec[wi];

  if (raw) {   // [128 + 144 R] floats: mu, V [R][128], C [16][R]
    float* r = raw + ((size_t)bi * hkv + kvh) * raw_floats(R);
    for (int i = lane; i < kD; i += 64) r[i] = sm.mu[i];
    for (int i = lane; i < R * kD; i += 64) r[kD + i] = sm.V[i >> 7][i & 127];
    for (int i = lane; i < kB * R; i += 64) r[kD + R * kD + i] = sm.u.q.C[i / R][i % R];
  }
}

template <int R>
hipError_t launch_build_r(const uint16_t* k_cache, int64_t block_stride, int64_t head_stride,
                          int64_t token_stride, const BlockSource& src, dim3 grid,
                          int32_t n_blocks, int32_t num_blocks, int32_t hkv, uint8_t* summaries,
                          float* raw_debug, const float* basis, hipStream_t stream) {
  hipLaunchKernelGGL(build_kernel<R>, grid, dim3(64), 0, stream, k_cache, block_stride,
                     head_stride, token_stride, src, n_blocks, num_blocks, hkv, summaries,
                     raw_debug, basis);
  return hipGetLastError();
}

hipError_t launch_build_any(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                            int64_t head_stride, int64_t token_stride, const BlockSource& src,
                            dim3 grid, int32_t n_blocks, int32_t num_blocks, int32_t hkv,
                            uint8_t* summaries, float* raw_debug, const float* basis,
                            hipStream_t stream) {
  switch (rank) {
    case 4:
      return launch_build_r<4>(k_cache, block_stride, head_stride, token_stride, src, grid,
                               n_blocks, num_blocks, hkv, summaries, raw_debug, basis, stream);
    case 8:
      return launch_build_r<8>(k_cache, block_stride, head_stride, token_stride, src, grid,
                               n_blocks, num_blocks, hkv, summaries, raw_debug, basis, stream);
    case 16:
      return launch_build_r<16>(k_cache, block_stride, head_stride, token_stride, src, grid,
                                n_blocks, num_blocks, hkv, summaries, raw_debug, basis, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_build(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                        int64_t head_stride, int64_t token_stride, const int32_t* block_ids,
                        int32_t n_blocks, int32_t num_blocks, int32_t hkv, uint8_t* summaries,
                        float* raw_debug, hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  BlockSource src{block_ids, nullptr, nullptr, 0, false, 0, 0};
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src,
                          dim3(n_blocks, hkv), n_blocks, num_blocks, hkv, summaries, raw_debug,
                          nullptr, stream);
}

hipError_t launch_build_basis(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                              int64_t head_stride, int64_t token_stride,
                              const int32_t* block_ids, int32_t n_blocks, int32_t num_blocks,
                              int32_t hkv, const float* basis, uint8_t* summaries,
                              hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  BlockSource src{block_ids, nullptr, nullptr, 0, false, 0, 0};
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src,
                          dim3(n_blocks, hkv), n_blocks, num_blocks, hkv, summaries, nullptr,
                          basis, stream);
}

hipError_t launch_finalize(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                           int64_t head_stride, int64_t token_stride, const int32_t* block_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                           int32_t num_blocks, int32_t hkv, uint8_t* summaries, int32_t n_layers,
                           int64_t k_layer_stride, int64_t summ_layer_stride,
                           hipStream_t stream) {
  BlockSource src{nullptr, seq_lens, block_table, max_pages, true, k_layer_stride,
                  summ_layer_stride};
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src,
                          dim3(batch, hkv, n_layers), batch, num_blocks, hkv, summaries, nullptr,
                          nullptr, stream);
}

}  // namespace locks
