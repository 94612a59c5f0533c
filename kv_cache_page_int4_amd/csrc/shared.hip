// The shared low-rank basis that the LOCKS pages contrast their page-local
// basis with (LOCKS explainer, technical summary sec. 1 and sec. 3,
// Proposition 1: one fixed, query-independent rank-r projection for all
// pages is blind to what varies inside a page).  It is the top-r eigenvectors
// of the page deviations pooled over many pages:
//   S = sum_j X_j^T X_j,   X_j = K_j - 1 mu_j^T  (each page centred on itself),
// and summaries built in it (builder with a given basis) feed the unchanged
// scorer and selection: the shared-basis selector, at the same state size.
//
// Two kernels, both off the decode path.
//  * scatter_kernel: workgroup (chunk, KV head) sums X_j^T X_j over a run of
//    pages of the block list.  256 threads, each owning an 8x8 tile of the
//    128x128 sum in registers; a page's keys go through LDS (centred there),
//    and the next page's keys are loaded while the current one is folded in.
//    Partial sums are written per chunk and added in chunk order later, so
//    the result does not depend on scheduling.
//  * eigen_kernel: one 1024-thread workgroup per KV head adds the partials
//    and runs cyclic Jacobi on the 128x128 matrix in LDS with round-robin
//    ordering (64 disjoint rotations per round, 127 rounds per sweep; each
//    round applies J^T A J and V <- V J), until the off-diagonal mass is below
//    1e-10 of the total (at most 24 sweeps).  The top-r eigenvectors
//    (descending eigenvalue, ties to the lower index) are normalized and
//    signed like a page's basis (largest-|entry| component positive, lowest
//    index on ties).
#include "locks_device.h"
#include "locks_internal.h"

#include <algorithm>

namespace locks {

namespace {

constexpr int kScatThreads = 256;
constexpr int kEigThreads = 1024;
constexpr int kEigMaxSweeps = 24;

__global__ __launch_bounds__(kScatThreads) void scatter_kernel(
    const uint16_t* __restrict__ kc, int64_t bs, int64_t hs, int64_t ts,
    const int32_t* __restrict__ block_ids, int32_t n_blocks, int32_t num_blocks,
    int32_t per_chunk, float* __restrict__ part) {
  const int chunk = blockIdx.x, kvh = blockIdx.y, n_chunks = gridDim.x;
  const int tid = threadIdx.x;
  __shared__ float X[kB][kD + 4];
  const int i0 = 8 * (tid >> 4), j0 = 8 * (tid & 15);   // this thread's tile of S
  const int lt = tid >> 4, ld = 8 * (tid & 15);         // this thread's 8 keys of a page
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;

  const int p0 = chunk * per_chunk, p1 = min(n_blocks, p0 + per_chunk);
  // keys of page p (zero for an out-of-range block id, which adds nothing)
  auto load = [&](int p) -> uint4 {
    const int blk = block_ids[p];
    if ((unsigned)blk >= (unsigned)num_blocks) return make_uint4(0u, 0u, 0u, 0u);
    return *reinterpret_cast<const uint4*>(kc + (size_t)blk * bs + (size_t)kvh * hs +
                                           (size_t)lt * ts + ld);
  };
  uint4 nxt = (p0 < p1) ? load(p0) : make_uint4(0u, 0u, 0u, 0u);
  for (int p = p0; p < p1; ++p) {
    const uint4 cur = nxt;
    if (p + 1 < p1) nxt = load(p + 1);
    const uint32_t w[4] = {cur.x, cur.y, cur.z, cur.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      X[lt][ld + 2 * e] = bf16_lo(w[e]);
      X[lt][ld + 2 * e + 1] = bf16_hi(w[e]);
    }
    __syncthreads();
    if (tid < kD) {   // centre dimension tid on the page's own mean
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < kB; ++t) m += X[t][tid];
      m *= 1.f / kB;
#pragma unroll
      for (int t = 0; t < kB; ++t) X[t][tid] -= m;
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 0; t < kB; ++t) {
      float xi[8], xj[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        xi[a] = X[t][i0 + a];
        xj[a] = X[t][j0 + a];
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(xi[a], xj[b], acc[a][b]);
    }
    __syncthreads();   // X is rewritten by the next page
  }
  float* dst = part + ((size_t)kvh * n_chunks + chunk) * kD * kD;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    float4* row = reinterpret_cast<float4*>(dst + (size_t)(i0 + a) * kD + j0);
    row[0] = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
    row[1] = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
  }
}

// Sum over the workgroup (all threads receive it).
__device__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return s;
}

struct EigSmem {
  float A[kD][kD + 1];   // the matrix, rotated towards diagonal
  float V[kD][kD + 1];   // accumulated rotations: eigenvectors as columns
  int p[kD / 2], q[kD / 2];
  float c[kD / 2], s[kD / 2];
  float red[kEigThreads / 64];
  int order[kD];
};

__global__ __launch_bounds__(kEigThreads) void eigen_kernel(const float* __restrict__ part,
                                                            int32_t n_chunks, int32_t rank,
                                                            float* __restrict__ basis,
                                                            float* __restrict__ eigvals) {
  __shared__ EigSmem sm;
  const int kvh = blockIdx.x, tid = threadIdx.x;
  const float* src = part + (size_t)kvh * n_chunks * kD * kD;
  for (int e = tid; e < kD * kD; e += kEigThreads) {
    float v = 0.f;
    for (int c = 0; c < n_chunks; ++c) v += src[(size_t)c * kD * kD + e];
    const int i = e >> 7, j = e & (kD - 1);
    sm.A[i][j] = v;
    sm.V[i][j] = (i == j) ? 1.f : 0.f;
  }
  __syncthreads();

  for (int sweep = 0; sweep < kEigMaxSweeps; ++sweep) {
    float off = 0.f, tot = 0.f;
    for (int e = tid; e < kD * kD; e += kEigThreads) {
      const int i = e >> 7, j = e & (kD - 1);
      const float v = sm.A[i][j];
      tot = fmaf(v, v, tot);
      if (i != j) off = fmaf(v, v, off);
    }
    off = block_sum(off, sm.red);
    tot = block_sum(tot, sm.red);
    // off-norm 1e-5 of the total: about the floor of fp32 rotations on a
    // 128 x 128 matrix (uniform: every thread holds the sums)
    if (!(off > 1e-10f * tot)) break;

    for (int r = 0; r < kD - 1; ++r) {
      // round-robin pairing: position 0 holds index 0, position m >= 1 holds
      // 1 + (m - 1 + r) mod 127; pair k joins positions k and 127 - k
      if (tid < kD / 2) {
        const int k = tid;
        const int a = (k == 0) ? 0 : 1 + (k - 1 + r) % (kD - 1);
        const int b = 1 + (kD - 2 - k + r) % (kD - 1);
        const int p = min(a, b), q = max(a, b);
        const float app = sm.A[p][p], aqq = sm.A[q][q], apq = sm.A[p][q];
        float c = 1.f, s = 0.f;
        if (apq != 0.f) {
          const float theta = (aqq - app) / (2.f * apq);
          const float t = (fabsf(theta) > 1e15f)
                              ? 0.5f / theta
                              : copysignf(1.f, theta) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
          c = 1.f / sqrtf(t * t + 1.f);
          s = t * c;
        }
        sm.p[k] = p;
        sm.q[k] = q;
        sm.c[k] = c;
        sm.s[k] = s;
      }
      __syncthreads();
      // rows p, q of J^T A
      for (int e = tid; e < (kD / 2) * kD; e += kEigThreads) {
        const int k = e >> 7, j = e & (kD - 1);
        const int p = sm.p[k], q = sm.q[k];
        const float c = sm.c[k], s = sm.s[k];
        const float ap = sm.A[p][j], aq = sm.A[q][j];
        sm.A[p][j] = c * ap - s * aq;
        sm.A[q][j] = s * ap + c * aq;
      }
      __syncthreads();
      // columns p, q of (J^T A) J and of V J
      for (int e = tid; e < (kD / 2) * kD; e += kEigThreads) {
        const int k = e >> 7, i = e & (kD - 1);
        const int p = sm.p[k], q = sm.q[k];
        const float c = sm.c[k], s = sm.s[k];
        const float ap = sm.A[i][p], aq = sm.A[i][q];
        sm.A[i][p] = c * ap - s * aq;
        sm.A[i][q] = s * ap + c * aq;
        const float vp = sm.V[i][p], vq = sm.V[i][q];
        sm.V[i][p] = c * vp - s * vq;
        sm.V[i][q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }

  // descending eigenvalues, ties to the lower index
  if (tid < kD) {
    const float lj = sm.A[tid][tid];
    int rank = 0;
    for (int i = 0; i < kD; ++i) {
      const float li = sm.A[i][i];
      rank += (li > lj) || (li == lj && i < tid);
    }
    sm.order[rank] = tid;
    if (eigvals) eigvals[(size_t)kvh * kD + rank] = lj;
  }
  __syncthreads();
  // wave k < rank: basis vector k (lane owns entries lane and lane + 64)
  const int wave = tid >> 6, lane = tid & 63;
  if (wave < rank) {
    const int col = sm.order[wave];
    float v0 = sm.V[lane][col], v1 = sm.V[lane + 64][col];
    float n2 = v0 * v0 + v1 * v1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) n2 += __shfl_xor(n2, o);
    const float inv = (n2 > 0.f) ? 1.f / sqrtf(n2) : 0.f;
    v0 *= inv;
    v1 *= inv;
    float best = fabsf(v0), bval = v0;
    int bidx = lane;
    if (fabsf(v1) > best) {
      best = fabsf(v1);
      bval = v1;
      bidx = lane + 64;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ob = __shfl_xor(best, o), ov = __shfl_xor(bval, o);
      const int oi = __shfl_xor(bidx, o);
      if (ob > best || (ob == best && oi < bidx)) {
        best = ob;
        bval = ov;
        bidx = oi;
      }
    }
    if (bval < 0.f) {
      v0 = -v0;
      v1 = -v1;
    }
    float* out = basis + ((size_t)kvh * rank + wave) * kD;
    out[lane] = v0;
    out[lane + 64] = v1;
  }
}

}  // namespace

SharedPlan plan_shared(int32_t n_blocks) {
  SharedPlan pl;
  // at most kSharedMaxChunks partial sums per KV head, at least 64 pages each
  pl.n_chunks = std::max(1, std::min(kSharedMaxChunks, (n_blocks + 63) / 64));
  pl.per_chunk = (n_blocks + pl.n_chunks - 1) / pl.n_chunks;
  return pl;
}

hipError_t launch_shared_basis(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                               int64_t head_stride, int64_t token_stride,
                               const int32_t* block_ids, int32_t n_blocks, int32_t num_blocks,
                               int32_t hkv, float* partials, const SharedPlan& plan,
                               float* basis, float* eigvals, hipStream_t stream) {
  hipLaunchKernelGGL(scatter_kernel, dim3(plan.n_chunks, hkv), dim3(kScatThreads), 0, stream,
                     k_cache, block_stride, head_stride, token_stride, block_ids, n_blocks,
                     num_blocks, plan.per_chunk, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(eigen_kernel, dim3(hkv), dim3(kEigThreads), 0, stream, partials,
                     plan.n_chunks, rank, basis, eigvals);
  return hipGetLastError();
}

}  // namespace locks
