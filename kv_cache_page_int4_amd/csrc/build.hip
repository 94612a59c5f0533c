// Page-summary builder: runs when a page is finalized, off the decode path
// (LOCKS explainer, technical summary sec. 2, core mechanism: the centroid,
// a small eigendecomposition of the page's centered keys, the top-r
// eigenvectors and one coefficient vector per token; int4 basis, int8
// coefficients and centroid).
//
// One wave per four (page, KV head) items:
//  1. per page, load the 16x128 bf16 keys, centroid mu by DPP row sums,
//     X = K - mu in fp32;
//  2. Gram matrix X X^T (16x16) on the matrix cores (fp32 16x16x4);
//  3. cyclic Jacobi on the four Gram matrices at once, one per 16-lane row
//     of the wave: pairs (i, i^m) for m = 1..15 form 8 disjoint rotations
//     per step; lane i of a row holds row i of its page's matrix and of the
//     eigenvector matrix, in registers; a page whose off-diagonal mass is
//     below 1e-12 of its total is held from then on, and the sweeps stop
//     once every page is (at most 10);
//  4. per page, the top-r eigenpairs (descending, ties to the lower index)
//     give the basis v_k = X^T u_k normalized to unit length (the dual of the
//     d x d scatter's eigenproblem), zeroed when lambda_k <= 1e-5 lambda_1 or
//     when the page is constant to rounding;
//  5. sign: the largest-|entry| component of v_k is made positive (lowest dim
//     on ties); coefficients c_i = V^T x_i are projections on the unquantized
//     basis (C = X V on the matrix cores, fp32 16x16x4);
//  6. symmetric quantization with fp16 scales (max|x|/7 for the basis,
//     max|x|/127 for coefficients and centroid, round half to even) and
//     packing into the 832-byte record.
// With a given basis (the shared-basis selector the pages contrast LOCKS
// with), steps 2-5 are replaced by that basis, one page per wave: the record
// keeps the page's own centroid and coefficients c_i = V^T x_i in the given
// basis.
#include <utility>

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

// Buffers of the basis, coefficient and packing phases of one page-head
// (phases 4-6), in LDS.
template <int R>
struct PackSmem {
  float V[R][kD + 4] __attribute__((aligned(16)));   // unquantized basis, [k][d]
  float mu[kD] __attribute__((aligned(16)));   // centroid
  float C[kB][R];          // unquantized coefficients
  int8_t vq[R][kD];
  uint32_t rec[RecLayout<R>::kBytes / 4];
};

// Which blocks a workgroup summarizes: entries of a list, or (for
// incremental finalization) for each sequence the last full page when that
// sequence's length is a positive multiple of the page size -- the page that
// the newest token just completed.
struct BlockSource {
  const int32_t* block_ids;    // list mode: [n]
  const int32_t* seq_lens;     // finalize mode: [batch]
  const int32_t* block_table;  // finalize mode: [batch][max_pages]
  int32_t max_pages;
  bool from_seq;
  int64_t k_layer_stride;      // finalize mode: layer blockIdx.z of the caches
  int64_t summ_layer_stride;
};

// Block of item bi (list entry or sequence), -1 when there is none or it is
// out of range.
__device__ __forceinline__ int item_block(const BlockSource& src, int bi, int n_items,
                                          int num_blocks) {
  if (bi >= n_items) return -1;
  int blk;
  if (src.from_seq) {
    const int seq = src.seq_lens[bi];
    const int j = seq / kB - 1;
    blk = (seq > 0 && seq % kB == 0 && j < src.max_pages)
              ? src.block_table[(size_t)bi * src.max_pages + j] : -1;
  } else {
    blk = src.block_ids[bi];
  }
  return ((unsigned)blk < (unsigned)num_blocks) ? blk : -1;
}

// ---- 1-2. one page-head's keys: centroid mu (to LDS when mu is given), and
// with GRAM the Gram matrix of the deviations (LDS, symmetrized).  Returns the keys' squared
// norm (wave-uniform).  Lane (t = token lane % 16, g = lane / 16) holds dims
// 32g .. 32g + 31 of token t.
template <bool GRAM>
__device__ __forceinline__ float centre_and_gram(const uint16_t* kpage, int64_t ts, float* mu,
                                                 float (*G)[kB + 1]) {
  const int lane = threadIdx.x;
  const int t = lane & 15, g = lane >> 4;
  const uint16_t* kp = kpage + (size_t)t * ts + 32 * g;
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
    if (mu && t == 0) mu[32 * g + e] = m;
  }
  ksq = wave_sum(ksq);
  if constexpr (GRAM) {
    // Gram matrix on the matrix cores: K index (step s, group g) = dim 32g+s
    f32x4v gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 32; ++s) gacc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], x[s], gacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) G[4 * g + r][t] = gacc[r];
    __syncthreads();
    // symmetrize (the product is symmetric up to rounding order)
    for (int i = lane; i < kB * kB; i += 64) {
      const int a = i >> 4, b = i & 15;
      if (a < b) {
        const float v = 0.5f * (G[a][b] + G[b][a]);
        G[a][b] = v;
        G[b][a] = v;
      }
    }
  }
  __syncthreads();
  return ksq;
}

// ---- 3. cyclic Jacobi, one 16x16 matrix per 16-lane group ----
// A step m (1..15) rotates the 8 disjoint index pairs (i, i ^ m).  Lane i of
// a group holds row i of G and of the eigenvector matrix U in XOR order:
// slot c holds column i ^ c, so the diagonal is slot 0, the pair's
// off-diagonal element slot m, and the column pairs of a step are the slot
// pairs (c, c ^ m) in every lane.  Values of other rows come from lanes of
// the same group: lane i reads lane i ^ X.  Six of the fifteen XORs are one
// DPP move (1, 2, 3 within quads, 7 and 15 by the row's half and full
// mirrors, 8 by a rotation of the row by half its width); every other one is
// a quad XOR after the half mirror (4, 5, 6), the rotation by 8 (9, 10, 11)
// or the full mirror (12, 13, 14).  With DPP2 those take the two moves;
// otherwise they take one swizzle of the LDS unit in its xor-mask mode,
// which costs no VALU issue but has the latency of an LDS access.  Both
// move the same bits.
template <int X, bool DPP2>
__device__ __forceinline__ float swz(float v) {
  constexpr int kQuadXor[4] = {qp(0, 1, 2, 3), qp(1, 0, 3, 2), qp(2, 3, 0, 1), qp(3, 2, 1, 0)};
  if constexpr (X == 0) return v;
  else if constexpr (X <= 3) return dpp<kQuadXor[X]>(v);
  else if constexpr (X == 7) return dpp<kRowHalfMirror>(v);
  else if constexpr (X == 8) return dpp<kRowRor8>(v);
  else if constexpr (X == 15) return dpp<kRowMirror>(v);
  else if constexpr (!DPP2)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (X << 10) | 0x1F));
  else if constexpr (X < 7) return dpp<kQuadXor[X ^ 7]>(dpp<kRowHalfMirror>(v));
  else if constexpr (X < 12) return dpp<kQuadXor[X ^ 8]>(dpp<kRowRor8>(v));
  else return dpp<kQuadXor[X ^ 15]>(dpp<kRowMirror>(v));
}

// Column pair of slots (LO, LO ^ M) of T = G J and U' = U J.  The pair's
// rotation is held by lane i ^ LO; its first column is slot LO when this
// lane's row is first (bit kHb of i ^ LO is that of i), else slot LO ^ M,
// which the sign sg accounts for.
template <int M, int LO, bool DPP2>
__device__ __forceinline__ void jacobi_cols(float (&a)[kB], float (&u)[kB], float (&tr)[kB],
                                            float c, float s, float sg) {
  constexpr int kHb = 31 - __builtin_clz(M);
  if constexpr ((LO & (1 << kHb)) == 0) {
    constexpr int HI = LO ^ M;
    const float cc = swz<LO, DPP2>(c), ss = swz<LO, DPP2>(s) * sg;
    tr[LO] = fmaf(a[LO], cc, -(a[HI] * ss));
    tr[HI] = fmaf(a[HI], cc, a[LO] * ss);
    const float ul = u[LO], uh = u[HI];
    u[LO] = fmaf(ul, cc, -(uh * ss));
    u[HI] = fmaf(uh, cc, ul * ss);
  }
}

// Slot L of G' = J^T T: rows i and i ^ M, the partner's value of column
// i ^ L from its slot L ^ M.
template <int M, int L, bool DPP2>
__device__ __forceinline__ void jacobi_row(float (&a)[kB], const float (&tr)[kB], float c,
                                           float sr) {
  const float par = swz<M, DPP2>(tr[L ^ M]);
  a[L] = fmaf(c, tr[L], -(sr * par));
}

template <int M, bool DPP2, int... L>
__device__ __forceinline__ void jacobi_step(float (&a)[kB], float (&u)[kB], int i, bool done,
                                            std::integer_sequence<int, L...>) {
  constexpr int kHb = 31 - __builtin_clz(M);
  // this lane's row is the pair's first (lower) index
  const bool first = !(i & (1 << kHb));
  // the pair's rotation, computed alike in both of its lanes
  const float d_par = swz<M, DPP2>(a[0]), o_par = swz<M, DPP2>(a[M]);
  const float app = first ? a[0] : d_par, aqq = first ? d_par : a[0];
  const float gpq = first ? a[M] : o_par, gqp = first ? o_par : a[M];
  float c, s;
  jacobi_rot(app, 0.5f * (gpq + gqp), aqq, c, s);
  // a page that has converged turns by the identity: its diagonal and
  // eigenvectors stay what they were when it converged
  c = done ? 1.f : c;
  s = done ? 0.f : s;
  const float sg = first ? 1.f : -1.f;
  float tr[kB];
  (jacobi_cols<M, L, DPP2>(a, u, tr, c, s, sg), ...);
  (jacobi_row<M, L, DPP2>(a, tr, c, s * sg), ...);
  a[M] = 0.f;   // the pair's off-diagonal element, zero by construction
}

template <bool DPP2, int... M>
__device__ __forceinline__ void jacobi_sweep(float (&a)[kB], float (&u)[kB], int i, bool done,
                                             std::integer_sequence<int, M...>) {
  (jacobi_step<M + 1, DPP2>(a, u, i, done, std::make_integer_sequence<int, kB>{}), ...);
}

// Whether eigenvalue i ^ C ranks before eigenvalue i (li, held by lane i):
// descending order, ties to the lower index.
template <int C>
__device__ __forceinline__ int ranks_before(float li, int i) {
  const float lj = swz<C, true>(li);
  return (lj > li) || (lj == li && (i ^ C) < i);
}

// Column i ^ C of U (slot C of lane i's row) goes to column rank(i ^ C) of
// the top-R eigenvector matrix when that rank is below R.
template <int R, int C>
__device__ __forceinline__ void put_top_column(float (*Ut)[R], const float (&u)[kB], int rank,
                                               int i) {
  const int rj = __float_as_int(swz<C, true>(__int_as_float(rank)));
  if (rj < R) Ut[i][rj] = u[C];
}

// Eigenvalues a[0] of the 16 lanes of a group, ranked; the top R of them and
// their eigenvectors (columns of U, lane i holding row i in XOR order) go
// to lam[0 .. R) and Ut[.][0 .. R) in descending order.
template <int R, int... C>
__device__ __forceinline__ void store_top_eigenpairs(const float (&a)[kB], const float (&u)[kB],
                                                     int i, float* lam, float (*Ut)[R],
                                                     std::integer_sequence<int, C...>) {
  const float li = a[0];
  const int rank = (ranks_before<C + 1>(li, i) + ...);
  put_top_column<R, 0>(Ut, u, rank, i);
  (put_top_column<R, C + 1>(Ut, u, rank, i), ...);
  if (rank < R) lam[rank] = li;
}

// ---- 4. the basis from the top-R eigenpairs (lam[k], column k of U, in
// descending order): v_k = X^T u_k / |X^T u_k|, zero below the floors; sign
// by the largest-|entry| component.  Lane owns dims 2 lane, 2 lane + 1; it
// forms the centroid of those dims from the keys it reads, summing the 16
// tokens in the order of the butterfly of phase 1 (pairs, quads, eights,
// halves), so mu is the same value bit for bit, and leaves it in pk.mu.
template <int R, typename KeyPair>
__device__ __forceinline__ void basis_from_eig(const float* lam, const float (*U)[R], float ksq,
                                               KeyPair key_pair, PackSmem<R>& pk) {
  const int lane = threadIdx.x;
  const int d0 = 2 * lane;
  const float lam1 = lam[0];
  const bool page_has_basis = lam1 > kEpsConst * ksq;
  float2 xr[kB];
#pragma unroll
  for (int tt = 0; tt < kB; ++tt) {
    const uint32_t kw = key_pair(tt, d0);
    xr[tt] = make_float2(bf16_lo(kw), bf16_hi(kw));
  }
  float2 s[kB];
#pragma unroll
  for (int tt = 0; tt < kB; ++tt) s[tt] = xr[tt];
#pragma unroll
  for (int w = 1; w < kB; w *= 2) {
#pragma unroll
    for (int tt = 0; tt < kB; tt += 2 * w) {
      s[tt].x += s[tt + w].x;
      s[tt].y += s[tt + w].y;
    }
  }
  const float mu0 = s[0].x * (1.f / 16.f), mu1 = s[0].y * (1.f / 16.f);
  pk.mu[d0] = mu0;
  pk.mu[d0 + 1] = mu1;
#pragma unroll
  for (int tt = 0; tt < kB; ++tt) {
    xr[tt].x -= mu0;
    xr[tt].y -= mu1;
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool keep = page_has_basis && (lam[k] > kTau * lam1);
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int tt = 0; tt < kB; ++tt) {
      const float uu = U[tt][k];
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
    pk.V[k][d0] = v0;
    pk.V[k][d0 + 1] = v1;
  }
  __syncthreads();
}

// ---- 5-6. coefficients c_ik = v_k . x_i on the unquantized basis, then
// symmetric quantization with fp16 scales and packing; the record is
// written to dst, and with raw the unquantized mu, V, C.
template <int R>
__device__ __forceinline__ void coeffs_and_pack(const uint16_t* kpage, int64_t ts, PackSmem<R>& pk,
                                                uint32_t* __restrict__ dst, float* raw) {
  using RL = RecLayout<R>;
  const float* mu = pk.mu;
  const int lane = threadIdx.x;
  const int d0 = 2 * lane;
  // C = X V on the matrix cores (fp32 16x16x4), laid out as the Gram of
  // phase 2: lane (t = lane % 16, g = lane / 16) brings token t's centred
  // dims 32g .. 32g + 31 as the A operand and column t of V (basis vector
  // t, zero for t >= R) at the same dims as the B operand, one dim per step;
  // it ends holding C[4g + r][t], r = 0..3.
  {
    const int t = lane & 15, g = lane >> 4;
    const uint16_t* kp = kpage + (size_t)t * ts + 32 * g;
    const float* vrow = pk.V[t < R ? t : 0] + 32 * g;
    const float* mrow = mu + 32 * g;
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 kv = *reinterpret_cast<const uint4*>(kp + 8 * s);
      const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
      const float4 m0 = *reinterpret_cast<const float4*>(mrow + 8 * s);
      const float4 m1 = *reinterpret_cast<const float4*>(mrow + 8 * s + 4);
      const float4 v0 = *reinterpret_cast<const float4*>(vrow + 8 * s);
      const float4 v1 = *reinterpret_cast<const float4*>(vrow + 8 * s + 4);
      const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1])) - m[e];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x, t < R ? v[e] : 0.f, acc, 0, 0, 0);
      }
    }
    if (t < R) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pk.C[4 * g + r][t] = acc[r];
    }
  }
  __syncthreads();

  // centroid
  const float mu0 = mu[d0], mu1 = mu[d0 + 1];
  const float s_mu = fp16_scale(wave_max(fmaxf(fabsf(mu0), fabsf(mu1))), 127.f);
  const int mq0 = quant(mu0, s_mu, 127), mq1 = quant(mu1, s_mu, 127);
  // basis scales and codes
  float s_v[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float a = pk.V[k][d0], b2 = pk.V[k][d0 + 1];
    s_v[k] = fp16_scale(wave_max(fmaxf(fabsf(a), fabsf(b2))), 7.f);
    pk.vq[k][d0] = (int8_t)quant(a, s_v[k], 7);
    pk.vq[k][d0 + 1] = (int8_t)quant(b2, s_v[k], 7);
  }
  // coefficient scales: column k max over the 16 tokens
  float s_c[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const float a = (lane < 16) ? fabsf(pk.C[lane][k]) : 0.f;
    s_c[k] = fp16_scale(wave_max(a), 127.f);
  }
  __syncthreads();
  // record words: basis, coefficients, centroid, s_V, s_c, s_mu, zero
  uint8_t* mub = reinterpret_cast<uint8_t*>(&pk.rec[RL::kWMu]);
  mub[d0] = (uint8_t)(int8_t)mq0;
  mub[d0 + 1] = (uint8_t)(int8_t)mq1;
  for (int wi = lane; wi < 16 * R; wi += 64) {
    const int k = wi >> 4, w = wi & 15;
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = (uint32_t)pk.vq[k][8 * w + m] & 0xFu;
      const uint32_t hi = (uint32_t)pk.vq[k][8 * w + 4 + m] & 0xFu;
      word |= (lo | (hi << 4)) << (8 * m);
    }
    pk.rec[wi] = word;
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
      word |= ((uint32_t)(uint8_t)(int8_t)quant(pk.C[tk][kh + e], sce, 127)) << (8 * e);
    }
    pk.rec[RL::kWC + lane] = word;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      pk.rec[RL::kWSv + i] = fp16_bits(s_v[2 * i]) | (fp16_bits(s_v[2 * i + 1]) << 16);
      pk.rec[RL::kWSc + i] = fp16_bits(s_c[2 * i]) | (fp16_bits(s_c[2 * i + 1]) << 16);
    }
    pk.rec[RL::kWSmu] = fp16_bits(s_mu);
    for (int i = RL::kWSmu + 1; i < RL::kBytes / 4; ++i) pk.rec[i] = 0u;
  }
  __syncthreads();
  for (int wi = lane; wi < RL::kBytes / 4; wi += 64) dst[wi] = pk.rec[wi];

  if (raw) {   // [128 + 144 R] floats: mu, V [R][128], C [16][R]
    for (int i = lane; i < kD; i += 64) raw[i] = mu[i];
    for (int i = lane; i < R * kD; i += 64) raw[kD + i] = pk.V[i >> 7][i & 127];
    for (int i = lane; i < kB * R; i += 64) raw[kD + R * kD + i] = pk.C[i / R][i % R];
  }
  __syncthreads();   // the buffers are free for the next page-head
}

// Pages per workgroup of the eigen-solving builder: one per 16-lane group.
constexpr int kBuildPages = 4;

// Launches of at most this many workgroups use the DPP-only exchanges (one
// wave per SIMD of the 256 CUs or fewer: nothing hides a swizzle's latency);
// larger ones use the swizzles, which spare the VALU.  The two forms move the
// same bits, so the records are the same.
constexpr int64_t kDppOnlyMaxWorkgroups = 1024;

// Summaries of kBuildPages page-heads (items kBuildPages * blockIdx.x + p,
// KV head blockIdx.y) per one-wave workgroup: phases 1-2 page by page, the
// Jacobi sweeps of all four at once (16 lanes each, no lane duplicating
// another's work), then phases 4-6 page by page.  LDS: the Gram matrices
// until the sweeps have read them, then in the same bytes the packing
// buffers, reused from page to page; the top-r eigenvectors and eigenvalues
// of the four pages apart.  DPP2: the Jacobi's lane exchanges by DPP moves
// only.
template <int R, bool DPP2>
__global__ __launch_bounds__(64) void build_kernel(const uint16_t* __restrict__ kc, int64_t bs,
                                                   int64_t hs, int64_t ts, BlockSource src,
                                                   int32_t n_items, int32_t num_blocks,
                                                   int32_t hkv, uint8_t* __restrict__ summ,
                                                   float* __restrict__ raw) {
  using RL = RecLayout<R>;
  __shared__ union {
    float G[kBuildPages][kB][kB + 1];   // Gram matrices, until the sweeps have read them
    PackSmem<R> pk;                     // then the packing buffers, page by page
  } sm;
  __shared__ float Ut[kBuildPages][kB][R];   // top-R eigenvectors, columns in rank order
  __shared__ float lam[kBuildPages][R];      // their eigenvalues
  const int lane = threadIdx.x;
  const int kvh = blockIdx.y;
  kc += (size_t)blockIdx.z * src.k_layer_stride;
  summ += (size_t)blockIdx.z * src.summ_layer_stride;
  int blk[kBuildPages];
  bool any = false;
#pragma unroll
  for (int p = 0; p < kBuildPages; ++p) {
    blk[p] = item_block(src, kBuildPages * blockIdx.x + p, n_items, num_blocks);
    any |= blk[p] >= 0;
  }
  if (!any) return;   // whole workgroup, uniform

  // ---- 1-2. per page: Gram matrix of the centred keys (a zero matrix for
  // an absent page, which the sweeps leave as it is) ----
  float ksq[kBuildPages];
#pragma unroll
  for (int p = 0; p < kBuildPages; ++p) {
    ksq[p] = 0.f;
    if (blk[p] >= 0) {
      ksq[p] = centre_and_gram<true>(kc + (size_t)blk[p] * bs + (size_t)kvh * hs, ts, nullptr,
                                     sm.G[p]);
    } else {
      for (int i = lane; i < kB * (kB + 1); i += 64) (&sm.G[p][0][0])[i] = 0.f;
    }
  }
  __syncthreads();

  // ---- 3. Jacobi, page lane / 16 in lanes 16 (lane / 16) .. +15 ----
  {
    const int grp = lane >> 4, i = lane & 15;
    float a[kB], u[kB];
#pragma unroll
    for (int c = 0; c < kB; ++c) {
      a[c] = sm.G[grp][i][i ^ c];
      u[c] = (c == 0) ? 1.f : 0.f;
    }
    // whether this lane's page has converged (the same in all 16 lanes of a
    // page): its off-diagonal mass is below 1e-12 of the total (off-norm
    // 1e-6 relative: far below what the codes and fp16 scales resolve).  The
    // sweeps go on until all four pages have; a page that converged earlier
    // is held where it converged, so a record does not depend on the pages
    // that share its wave.
    bool done = false;
    for (int sweep = 0; sweep < kSweeps; ++sweep) {
      jacobi_sweep<DPP2>(a, u, i, done, std::make_integer_sequence<int, kB - 1>{});
      float off = 0.f;
#pragma unroll
      for (int c = 1; c < kB; ++c) off = fmaf(a[c], a[c], off);
      const float tot = row_sum16(fmaf(a[0], a[0], off));
      off = row_sum16(off);
      done = done || !(off > 1e-12f * tot);
      if (__all(done)) break;
    }
    store_top_eigenpairs<R>(a, u, i, lam[grp], Ut[grp], std::make_integer_sequence<int, kB - 1>{});
  }
  __syncthreads();   // the Gram matrices are read: the LDS takes the packing buffers

  // ---- 4-6. per page: basis, coefficients, quantization, record ----
#pragma unroll 1
  for (int p = 0; p < kBuildPages; ++p) {
    if (blk[p] < 0) continue;   // uniform
    const uint16_t* kpage = kc + (size_t)blk[p] * bs + (size_t)kvh * hs;
    auto key_pair = [&](int tt, int d) {
      return *reinterpret_cast<const uint32_t*>(kpage + (size_t)tt * ts + d);
    };
    basis_from_eig<R>(lam[p], Ut[p], ksq[p], key_pair, sm.pk);
    uint32_t* dst =
        reinterpret_cast<uint32_t*>(summ + ((size_t)kvh * num_blocks + blk[p]) * RL::kBytes);
    float* r = raw ? raw + ((size_t)(kBuildPages * blockIdx.x + p) * hkv + kvh) * raw_floats(R)
                   : nullptr;
    coeffs_and_pack<R>(kpage, ts, sm.pk, dst, r);
  }
}

// Summaries in a given basis (the shared-basis selector the pages contrast
// LOCKS with): one page-head per one-wave workgroup, phases 1, 5 and 6 with
// V = the given basis of KV head blockIdx.y.
template <int R>
__global__ __launch_bounds__(64) void build_basis_kernel(const uint16_t* __restrict__ kc,
                                                         int64_t bs, int64_t hs, int64_t ts,
                                                         BlockSource src, int32_t n_items,
                                                         int32_t num_blocks,
                                                         uint8_t* __restrict__ summ,
                                                         const float* __restrict__ basis) {
  using RL = RecLayout<R>;
  __shared__ PackSmem<R> pk;
  const int lane = threadIdx.x;
  const int kvh = blockIdx.y;
  const int blk = item_block(src, blockIdx.x, n_items, num_blocks);
  if (blk < 0) return;   // whole workgroup, uniform
  const uint16_t* kpage = kc + (size_t)blk * bs + (size_t)kvh * hs;
  centre_and_gram<false>(kpage, ts, pk.mu, nullptr);
  const int d0 = 2 * lane;
  const float* bk = basis + (size_t)kvh * R * kD;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    pk.V[k][d0] = bk[k * kD + d0];
    pk.V[k][d0 + 1] = bk[k * kD + d0 + 1];
  }
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(summ + ((size_t)kvh * num_blocks + blk) * RL::kBytes);
  coeffs_and_pack<R>(kpage, ts, pk, dst, nullptr);
}

template <int R>
hipError_t launch_build_r(const uint16_t* k_cache, int64_t block_stride, int64_t head_stride,
                          int64_t token_stride, const BlockSource& src, int32_t n_items,
                          int32_t hkv, int32_t n_layers, int32_t num_blocks, uint8_t* summaries,
                          float* raw_debug, const float* basis, hipStream_t stream) {
  if (basis) {
    hipLaunchKernelGGL(build_basis_kernel<R>, dim3(n_items, hkv, n_layers), dim3(64), 0, stream,
                       k_cache, block_stride, head_stride, token_stride, src, n_items,
                       num_blocks, summaries, basis);
  } else {
    const int32_t wgs = (n_items + kBuildPages - 1) / kBuildPages;
    const bool dpp_only = (int64_t)wgs * hkv * n_layers <= kDppOnlyMaxWorkgroups;
    auto* kernel = dpp_only ? build_kernel<R, true> : build_kernel<R, false>;
    hipLaunchKernelGGL(kernel, dim3(wgs, hkv, n_layers), dim3(64), 0, stream, k_cache,
                       block_stride, head_stride, token_stride, src, n_items, num_blocks, hkv,
                       summaries, raw_debug);
  }
  return hipGetLastError();
}

hipError_t launch_build_any(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                            int64_t head_stride, int64_t token_stride, const BlockSource& src,
                            int32_t n_items, int32_t hkv, int32_t n_layers, int32_t num_blocks,
                            uint8_t* summaries, float* raw_debug, const float* basis,
                            hipStream_t stream) {
  switch (rank) {
    case 4:
      return launch_build_r<4>(k_cache, block_stride, head_stride, token_stride, src, n_items,
                               hkv, n_layers, num_blocks, summaries, raw_debug, basis, stream);
    case 8:
      return launch_build_r<8>(k_cache, block_stride, head_stride, token_stride, src, n_items,
                               hkv, n_layers, num_blocks, summaries, raw_debug, basis, stream);
    case 16:
      return launch_build_r<16>(k_cache, block_stride, head_stride, token_stride, src, n_items,
                                hkv, n_layers, num_blocks, summaries, raw_debug, basis, stream);
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
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src, n_blocks,
                          hkv, 1, num_blocks, summaries, raw_debug, nullptr, stream);
}

hipError_t launch_build_basis(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                              int64_t head_stride, int64_t token_stride,
                              const int32_t* block_ids, int32_t n_blocks, int32_t num_blocks,
                              int32_t hkv, const float* basis, uint8_t* summaries,
                              hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  BlockSource src{block_ids, nullptr, nullptr, 0, false, 0, 0};
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src, n_blocks,
                          hkv, 1, num_blocks, summaries, nullptr, basis, stream);
}

hipError_t launch_finalize(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                           int64_t head_stride, int64_t token_stride, const int32_t* block_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                           int32_t num_blocks, int32_t hkv, uint8_t* summaries, int32_t n_layers,
                           int64_t k_layer_stride, int64_t summ_layer_stride,
                           hipStream_t stream) {
  BlockSource src{nullptr, seq_lens, block_table, max_pages, true, k_layer_stride,
                  summ_layer_stride};
  return launch_build_any(rank, k_cache, block_stride, head_stride, token_stride, src, batch,
                          hkv, n_layers, num_blocks, summaries, nullptr, nullptr, stream);
}

}  // namespace locks
