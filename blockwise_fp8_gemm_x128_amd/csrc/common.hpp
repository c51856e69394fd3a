// Shared host validation and device helpers for libpuro (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "puro.h"

namespace puro {

// ---------------------------------------------------------------- host-side validation
constexpr int64_t kGroup = 128;
// Largest accepted dimension; keeps every element offset far inside int64 and every grid
// inside hipLaunchKernel's 32-bit limits.
constexpr int64_t kMaxDim = int64_t(1) << 24;

inline bool dim_ok(int64_t d) { return d >= 0 && d <= kMaxDim && d % kGroup == 0; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks one tensor pointer: NULL is only accepted for an empty tensor.
inline puro_status check_ptr(const void* p, bool empty) {
  if (empty) return PURO_OK;
  if (p == nullptr) return PURO_ERR_NULL;
  if (!aligned16(p)) return PURO_ERR_ALIGN;
  return PURO_OK;
}

inline puro_status launch_status() {
  return hipGetLastError() == hipSuccess ? PURO_OK : PURO_ERR_LAUNCH;
}

#define PURO_TRY(expr)                   \
  do {                                   \
    puro_status st_ = (expr);            \
    if (st_ != PURO_OK) return st_;      \
  } while (0)

// ---------------------------------------------------------------- device helpers
// bf16 <-> fp32: bf16 is the high half of a binary32, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16 packed in one dword (lo in bits 0-15), round to nearest even: gfx950
// converts both in one v_cvt_pk_bf16_f32 (checked on MI355X against the integer
// round-to-nearest-even rule, denormals included).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Four fp32 values, already multiplied by the group's reciprocal scale, to four OCP E4M3 bytes
// (byte i holds value i). The clamp to +-448 is the contract's saturation step; the convert
// rounds to nearest even and keeps the sign of zero.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return static_cast<uint32_t>(v);
}

// Scale and reciprocal of a group from its max magnitude: s = amax/448, r = 448/amax, each a
// single correctly rounded fp32 division; an all-zero group gets s = r = 1.
__device__ __forceinline__ void group_scale(float amax, float& s, float& r) {
  if (amax == 0.0f) {
    s = 1.0f;
    r = 1.0f;
  } else {
    s = amax / 448.0f;
    r = 448.0f / amax;
  }
}

// Cross-lane maxima of non-negative fp32 values (magnitudes), in registers: for such values the
// order of the bit patterns as unsigned integers is the order of the values, so an integer max
// of the patterns is exact and needs no NaN handling (inputs are finite by contract).
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}
// Max over the 16 lanes of each row of the wave (lanes 16k .. 16k+15): swap neighbours, swap
// pairs, mirror halves of 8, mirror the row.
__device__ __forceinline__ float row16_max(float m) {
  uint32_t u = __float_as_uint(m);
  u = umax32(u, dpp<0xB1>(u));   // quad_perm [1,0,3,2]
  u = umax32(u, dpp<0x4E>(u));   // quad_perm [2,3,0,1]
  u = umax32(u, dpp<0x141>(u));  // row_half_mirror
  u = umax32(u, dpp<0x140>(u));  // row_mirror
  return __uint_as_float(u);
}
// Max over lanes l, l^16, l^32, l^48 (across the four rows of the wave).
__device__ __forceinline__ float across_rows_max(float m) {
  uint32_t u = __float_as_uint(m);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = umax32(p16[0], p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(umax32(p32[0], p32[1]));
}
// Max over lanes l, l^8, l^16, ..., l^56 (the eight lanes of a wave that share l mod 8).
__device__ __forceinline__ float stride8_max(float m) {
  uint32_t u = __float_as_uint(m);
  u = umax32(u, dpp<0x128>(u));  // row_ror:8 (lane l and l^8 within a row)
  return across_rows_max(__uint_as_float(u));
}

// Power-of-two scale of a group: s = 2^e for the least integer e with 448 * 2^e >= amax, raised
// to -127 when smaller, and r = 2^-e exactly, so x * r is exact; an all-zero group gets
// s = r = 1. With amax = (1 + f) * 2^(E - 127) (E the biased exponent field, f the fraction)
// and 448 = 1.75 * 2^8: e = E - 135 when 1 + f <= 1.75, else E - 134. A subnormal amax lands
// far below -127 and is raised to it. Finite bf16 inputs keep e <= 120, so 2^-e is a normal
// fp32; s = 2^-127 is the fp32 subnormal 0x00400000.
__device__ __forceinline__ void group_scale_pow2(float amax, float& s, float& r) {
  const uint32_t u = __float_as_uint(amax);
  int e = static_cast<int>(u >> 23) - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  e = e < -127 ? -127 : e;
  if (amax == 0.0f) e = 0;
  s = e >= -126 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23)
                : __uint_as_float(0x00400000u);
  r = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

// The group scale rule a kernel is instantiated for.
template <bool kPow2>
__device__ __forceinline__ void scale_rule(float amax, float& s, float& r) {
  if constexpr (kPow2)
    group_scale_pow2(amax, s, r);
  else
    group_scale(amax, s, r);
}

}  // namespace puro
