// Device helpers shared by the LOCKS kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

constexpr int kD = 128;        // head dim
constexpr int kB = 16;         // tokens per page
constexpr int kR = 8;          // basis vectors per page
constexpr int kG = 4;          // query heads per KV head
constexpr int kRec = 832;      // bytes per summary record
constexpr int kOffV = 0, kOffC = 512, kOffMu = 640, kOffSv = 768, kOffSc = 784, kOffSmu = 800;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// DPP lane moves.  quad_perm selectors move values within groups of 4
// lanes; row_* selectors act within rows of 16 lanes.
constexpr int qp(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor4 = 0x124;   // rotate the 16 lanes of each row by 4
constexpr int kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of lane (4*(lane/4) + H) within each quad.
template <int H>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp<qp(H, H, H, H)>(x);
}

// Sum / max over the 16 lanes of each row, result in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<qp(1, 0, 3, 2)>(x);
  x += dpp<qp(2, 3, 0, 1)>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<qp(1, 0, 3, 2)>(x));
  x = fmaxf(x, dpp<qp(2, 3, 0, 1)>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two (max, sum) pairs of a base-2 log-sum-exp.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace locks
