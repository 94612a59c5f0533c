// Device helpers shared by the LOCKS kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

constexpr int kD = 128;        // head dim
constexpr int kB = 16;         // tokens per page
constexpr int kR = 8;          // basis vectors per page
constexpr int kRec = 832;      // bytes per summary record
constexpr int kOffV = 0, kOffC = 512, kOffMu = 640, kOffSv = 768, kOffSc = 784, kOffSmu = 800;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Pages of a sequence of `seq` tokens (clamped to its table) whose summaries
// are in use: every full page, or, when the newest page is pending, every
// page before the one that holds the newest token.  The tokens after them
// (0..15 of them, or 1..16 when pending) are attended in full.
__device__ __forceinline__ int summarized_pages(int seq, int pending) {
  return seq > 0 ? (seq - pending) / kB : 0;
}

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

// ---- cross-row exchange without LDS -------------------------------------------
// gfx950's row swaps: v_permlane16_swap exchanges rows 0<->1 and 2<->3 between
// its two operands, v_permlane32_swap the two halves.  Applied to two copies
// of x, every lane gets the pair (x at this lane's slot in the lower row or
// half, x at the same slot in the upper one): the same pair in both lanes.
__device__ __forceinline__ void swap16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  lo = r[0];
  hi = r[1];
}
__device__ __forceinline__ void swap32(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  lo = r[0];
  hi = r[1];
}

// Sum / max over the lanes l, l^16, l^32, l^48 (the same slot of the four
// rows); a + b == b + a, so the result equals a butterfly over lanes 16 and
// 32 apart bit for bit.
__device__ __forceinline__ float cross_rows_sum(float x) {
  float a, b;
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}
__device__ __forceinline__ float cross_rows_max(float x) {
  float a, b;
  swap16(x, a, b);
  x = fmaxf(a, b);
  swap32(x, a, b);
  return fmaxf(a, b);
}

// Whole-wave reductions, the result in every lane.
__device__ __forceinline__ float wave_sum_f(float x) { return cross_rows_sum(row_sum16(x)); }
__device__ __forceinline__ float wave_max_f(float x) { return cross_rows_max(row_max16(x)); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t x) {
  x += dpp_u<qp(1, 0, 3, 2)>(x);
  x += dpp_u<qp(2, 3, 0, 1)>(x);
  x += dpp_u<kRowHalfMirror>(x);
  x += dpp_u<kRowMirror>(x);
  uint32_t a, b;
  swap16(x, a, b);
  x = a + b;
  swap32(x, a, b);
  return a + b;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t x) {
  x = min(x, dpp_u<qp(1, 0, 3, 2)>(x));
  x = min(x, dpp_u<qp(2, 3, 0, 1)>(x));
  x = min(x, dpp_u<kRowHalfMirror>(x));
  x = min(x, dpp_u<kRowMirror>(x));
  uint32_t a, b;
  swap16(x, a, b);
  x = min(a, b);
  swap32(x, a, b);
  return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) {
  x = max(x, dpp_u<qp(1, 0, 3, 2)>(x));
  x = max(x, dpp_u<qp(2, 3, 0, 1)>(x));
  x = max(x, dpp_u<kRowHalfMirror>(x));
  x = max(x, dpp_u<kRowMirror>(x));
  uint32_t a, b;
  swap16(x, a, b);
  x = max(a, b);
  swap32(x, a, b);
  return max(a, b);
}

// (max, sum) pairs of a base-2 log-sum-exp merged over the whole wave.
// lse2_merge gives the same bits with its two operands exchanged, so every
// lane of a pair ends with the same value.
__device__ __forceinline__ void wave_lse2(float& m, float& s) {
  lse2_merge(m, s, dpp<qp(1, 0, 3, 2)>(m), dpp<qp(1, 0, 3, 2)>(s));
  lse2_merge(m, s, dpp<qp(2, 3, 0, 1)>(m), dpp<qp(2, 3, 0, 1)>(s));
  lse2_merge(m, s, dpp<kRowHalfMirror>(m), dpp<kRowHalfMirror>(s));
  lse2_merge(m, s, dpp<kRowMirror>(m), dpp<kRowMirror>(s));
  float ma, mb, sa, sb;
  swap16(m, ma, mb);
  swap16(s, sa, sb);
  m = ma;
  s = sa;
  lse2_merge(m, s, mb, sb);
  swap32(m, ma, mb);
  swap32(s, sa, sb);
  m = ma;
  s = sa;
  lse2_merge(m, s, mb, sb);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4 and 8 within each
// row, then the last lane of row 0 (of rows 0-1) is added to rows 1 and 3
// (2 and 3).  Lanes with no source take the old value 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_src(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_add_src<0x111, 0xF>(x);   // row_shr:1
  x += dpp_add_src<0x112, 0xF>(x);   // row_shr:2
  x += dpp_add_src<0x114, 0xF>(x);   // row_shr:4
  x += dpp_add_src<0x118, 0xF>(x);   // row_shr:8
  x += dpp_add_src<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_add_src<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace locks
