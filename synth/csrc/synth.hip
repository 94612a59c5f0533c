// Device-side synthetic inputs (same recipe as synth/host.py, Philox stream).
// Holds no part of the LOCKS method: only random keys, values and queries.
//
// Random numbers: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), written from its published
// definition; normals by the Box-Muller transform.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ void mulhilo(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  const uint64_t p = (uint64_t)a * (uint64_t)b;
  hi = (uint32_t)(p >> 32);
  lo = (uint32_t)p;
}

__device__ U4 philox(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(0xD2511F53u, c.x, hi0, lo0);
    mulhilo(0xCD9E8D57u, c.z, hi1, lo1);
    c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float uniform01(uint32_t v) {  // (0, 1)
  return ((float)(v >> 8) + 0.5f) * (1.0f / 16777216.0f);
}

// Four standard normals for counter c under key (k0, k1).
__device__ void normal4(U4 c, uint32_t k0, uint32_t k1, float out[4]) {
  const U4 r = philox(c, k0, k1);
  const float u1 = uniform01(r.x), u2 = uniform01(r.y), u3 = uniform01(r.z), u4 = uniform01(r.w);
  const float a = sqrtf(-2.f * logf(u1)), b = sqrtf(-2.f * logf(u3));
  const float t1 = 6.283185307179586f * u2, t2 = 6.283185307179586f * u4;
  out[0] = a * cosf(t1);
  out[1] = a * sinf(t1);
  out[2] = b * cosf(t2);
  out[3] = b * sinf(t2);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// purposes (third counter word, high byte)
enum : uint32_t { kCentroid = 1, kBasis = 2, kCoef = 3, kNoise = 4, kValue = 5, kQuery = 6, kCarrier = 7 };

__global__ void fill_q_kernel(uint16_t* q, int64_t n, uint32_t seed, uint32_t layer) {
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i4 >= n) return;
  float z[4];
  normal4(U4{(uint32_t)i4, (uint32_t)(i4 >> 32), kQuery << 24, 0u}, seed, layer, z);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (4 * i4 + e < n) q[4 * i4 + e] = to_bf16(z[e]);
}

// One wave per (logical page, KV head, sequence).
__global__ __launch_bounds__(64) void fill_pages_kernel(
    uint16_t* kc, uint16_t* vc, int64_t bs, int64_t hs, int64_t ts, const int32_t* block_table,
    const int32_t* seq_lens, int32_t max_pages, uint32_t seed, uint32_t layer, float noise_sd,
    int32_t coef_inv_k) {
  const int page = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int seq = seq_lens[b];
  const int n_pages = (seq + 15) / 16;
  if (page >= n_pages || page >= max_pages) return;
  const int valid = min(16, seq - 16 * page);
  const int blk = block_table[(size_t)b * max_pages + page];
  // counter words: (page, (b << 16) | kvh, purpose << 24 | index / 4, 0)
  const uint32_t c1 = ((uint32_t)b << 16) | (uint32_t)kvh;
  auto nrm4 = [&](uint32_t purpose, uint32_t idx4, float z[4]) {
    normal4(U4{(uint32_t)page, c1, (purpose << 24) | idx4, 0u}, seed, layer, z);
  };
  // lane owns dims 2*lane, 2*lane+1; draw 4 normals covering dims 4*(lane/2)..+3
  const int d0 = 2 * lane;
  auto pick2 = [&](uint32_t purpose, uint32_t base4, float& a, float& bb) {
    float z[4];
    nrm4(purpose, base4 + (uint32_t)(lane >> 1), z);
    a = z[2 * (lane & 1)];
    bb = z[2 * (lane & 1) + 1];
  };
  float cen0, cen1;
  pick2(kCentroid, 0, cen0, cen1);
  // Haar-random orthonormal u_1..u_8 by modified Gram-Schmidt of Gaussian columns
  float u0[8], u1[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float g0, g1;
    pick2(kBasis, 32u * k, g0, g1);
#pragma unroll
    for (int j = 0; j < k; ++j) {
      const float dot = wave_sum(g0 * u0[j] + g1 * u1[j]);
      g0 -= dot * u0[j];
      g1 -= dot * u1[j];
    }
    const float inv = 1.f / sqrtf(wave_sum(g0 * g0 + g1 * g1));
    u0[k] = g0 * inv;
    u1[k] = g1 * inv;
  }
  uint16_t* kp = kc + (size_t)blk * bs + (size_t)kvh * hs + d0;
  uint16_t* vp = vc + (size_t)blk * bs + (size_t)kvh * hs + d0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float n0, n1, w0, w1;
    pick2(kNoise, 32u * i, n0, n1);
    pick2(kValue, 32u * i, w0, w1);
    // coefficients a_ik of token i (the same draws in every lane)
    float z[8];
    nrm4(kCoef, 2u * i, z);
    nrm4(kCoef, 2u * i + 1u, z + 4);
    float k0 = cen0 + n0 * noise_sd, k1 = cen1 + n1 * noise_sd;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sd = coef_inv_k ? rsqrtf((float)(k + 1)) : 1.f / (float)(k + 1);
      k0 = fmaf(z[k] * sd, u0[k], k0);
      k1 = fmaf(z[k] * sd, u1[k], k1);
    }
    const bool ok = i < valid;
    const uint32_t kw = ok ? ((uint32_t)to_bf16(k0) | ((uint32_t)to_bf16(k1) << 16)) : 0u;
    const uint32_t vw = ok ? ((uint32_t)to_bf16(w0) | ((uint32_t)to_bf16(w1) << 16)) : 0u;
    *reinterpret_cast<uint32_t*>(kp + (size_t)i * ts) = kw;
    *reinterpret_cast<uint32_t*>(vp + (size_t)i * ts) = vw;
  }
}

// carriers: [n][5] = (sequence, kv head, logical page, token slot, query head)
__global__ __launch_bounds__(64) void plant_carriers_kernel(
    uint16_t* kc, int64_t bs, int64_t hs, int64_t ts, const int32_t* block_table,
    int32_t max_pages, const uint16_t* q, int32_t hq, const int32_t* carriers, int32_t n,
    uint32_t seed, uint32_t layer, float noise_sd) {
  const int c = blockIdx.x;
  if (c >= n) return;
  const int lane = threadIdx.x;
  const int32_t* cr = carriers + 5 * c;
  const int b = cr[0], kvh = cr[1], page = cr[2], slot = cr[3], h = cr[4];
  const int blk = block_table[(size_t)b * max_pages + page];
  const uint16_t* qh = q + ((size_t)b * hq + h) * 128;
  const float q0 = from_bf16(qh[2 * lane]), q1 = from_bf16(qh[2 * lane + 1]);
  const float inv = 3.f / sqrtf(wave_sum(q0 * q0 + q1 * q1));
  float z[4];
  normal4(U4{(uint32_t)c, 0u, (kCarrier << 24) | (uint32_t)(lane >> 1), 0u}, seed, layer, z);
  const float n0 = z[2 * (lane & 1)], n1 = z[2 * (lane & 1) + 1];
  uint16_t* kp = kc + (size_t)blk * bs + (size_t)kvh * hs + (size_t)slot * ts + 2 * lane;
  kp[0] = to_bf16(q0 * inv + n0 * noise_sd);
  kp[1] = to_bf16(q1 * inv + n1 * noise_sd);
}

// Plain streaming copy (16-byte words), used to calibrate byte counters.
__global__ void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Plain streaming read (16-byte words) reduced to one word per workgroup:
// the achievable HBM read bandwidth of this device.
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 1; o < 64; o <<= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

extern "C" {

int synth_read(const void* src, int64_t bytes, void* sink, int32_t blocks, void* stream) {
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

int synth_fill_q(void* q, int64_t n, uint32_t seed, uint32_t layer, void* stream) {
  const int64_t n4 = (n + 3) / 4;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(fill_q_kernel, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)q, n, seed, layer);
  return (int)hipGetLastError();
}

int synth_fill_pages(void* kc, void* vc, int64_t bs, int64_t hs, int64_t ts,
                     const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                     int32_t hkv, int32_t max_pages, uint32_t seed, uint32_t layer,
                     float noise_sd, int32_t coef_inv_k, void* stream) {
  hipLaunchKernelGGL(fill_pages_kernel, dim3(max_pages, hkv, batch), dim3(64), 0,
                     (hipStream_t)stream, (uint16_t*)kc, (uint16_t*)vc, bs, hs, ts, block_table,
                     seq_lens, max_pages, seed, layer, noise_sd, coef_inv_k);
  return (int)hipGetLastError();
}

int synth_plant_carriers(void* kc, int64_t bs, int64_t hs, int64_t ts,
                         const int32_t* block_table, int32_t max_pages, const void* q, int32_t hq,
                         const int32_t* carriers, int32_t n, uint32_t seed, uint32_t layer,
                         float noise_sd, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(plant_carriers_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream,
                     (uint16_t*)kc, bs, hs, ts, block_table, max_pages, (const uint16_t*)q, hq,
                     carriers, n, seed, layer, noise_sd);
  return (int)hipGetLastError();
}

int synth_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (uint4*)dst,
                     (const uint4*)src, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
