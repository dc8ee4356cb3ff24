// Internal helpers shared by the HIP sources of libqspec.so (not part of the
// C ABI).  gfx950 only: 64-lane wavefronts, MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "qspec.h"

namespace qspec {

// thread-local error text behind qspec_last_error()
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
qspec_status fail(qspec_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
const char* last_error();
qspec_status device_check();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

constexpr int kGroup = 128;

// ---------------------------------------------------------------- vector types
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- device math
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight packed two's-complement nibbles (codes k0..k7, k0 in bits 0-3) ->
// four words of bf16 pairs holding 136 + q: (k0,k4) (k1,k5) (k2,k6) (k3,k7).
// 0x4300 | u is the bf16 of 128 + u, and u = q + 8 is the nibble with its
// sign bit flipped, so every value is exact.
__device__ __forceinline__ void w4_to_bf16_biased(uint32_t p, uint32_t o[4]) {
  // nibble pair (k_j, k_{j+4}) masked into bits 0-3 / 16-19, then one XOR
  // flips the nibble sign bits (u = q + 8) and sets the 0x43 high bytes
  // (the compiler fuses each mask-and-XOR into one v_bitop3_b32)
  constexpr uint32_t mask = 0x000F000Fu, bias = 0x43084308u;
  o[0] = (p & mask) ^ bias;
  o[1] = ((p >> 4) & mask) ^ bias;
  o[2] = ((p >> 8) & mask) ^ bias;
  o[3] = ((p >> 12) & mask) ^ bias;
}
constexpr float kW4Bias = 136.0f;

// Eight natural-order bf16 values in four words -> the pair order of
// w4_to_bf16_biased: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ void bf16x8_interleave(const uint32_t x[4], uint32_t o[4]) {
  o[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);
  o[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);
}

// Eight packed nibbles -> two words of int8 holding 16 * q:
// lo = codes k0,k2,k4,k6 and hi = codes k1,k3,k5,k7 (byte i of each word).
__device__ __forceinline__ uint32_t w4_lo_x16(uint32_t p) { return (p << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t w4_hi_x16(uint32_t p) { return p & 0xF0F0F0F0u; }

// Fixed-order sum of eight natural-order bf16 values (four words).
__device__ __forceinline__ float bf16x8_sum(const uint32_t x[4]) {
  float a = bf16_lo(x[0]) + bf16_hi(x[0]);
  float b = bf16_lo(x[1]) + bf16_hi(x[1]);
  float c = bf16_lo(x[2]) + bf16_hi(x[2]);
  float d = bf16_lo(x[3]) + bf16_hi(x[3]);
  return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Wavefront reductions over DPP lane moves (no LDS round trip): each
// 16-lane row by swapping neighbours and pairs and rotating by 4 and 8 lanes,
// then the four rows' values (lanes 0, 16, 32, 48) read in a fixed order, so
// the result is a fixed function of the 64 inputs and every lane gets it.
// Every lane of the wavefront must be active.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum over the wavefront, the same value in every lane: each 16-lane row by
// DPP moves (lane 0 of the row keeps a fixed association), then the rows'
// sums (r0 + r1) + (r2 + r3).  Every lane must be active.
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<0xB1>(v);   // lane ^ 1
  v += dpp_f64<0x4E>(v);   // lane ^ 2
  v += dpp_f64<0x124>(v);  // row rotate 4
  v += dpp_f64<0x128>(v);  // row rotate 8
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Sum over each 16-lane row by DPP moves (swap neighbours, swap pairs,
// rotate the row by 4 and by 8); lane 0 of the row holds a fixed
// association of the row's 16 values.  Every lane of the row must be active.
__device__ __forceinline__ float row16_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
}


// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with one rounding: truncate to fp32 and set the lowest bit if
// anything was dropped (round to odd keeps the information a later rounding
// to nearest needs), then round fp32 -> bf16 to nearest even.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  float t = __double2float_rz(v);
  uint32_t u = __float_as_uint(t);
  if ((double)t != v) u |= 1u;
  return f32_to_bf16_rne(__uint_as_float(u));
}

// SwiGLU of one gate / up pair of fp32 GEMM outputs: bf16(silu(g) * u),
// silu(g) = g / (1 + exp(-g)), in fp64 with one rounding.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
  const double gd = g, ud = u;
  return f64_to_bf16_rne(gd / (1.0 + exp(-gd)) * ud);
}

// The code of v at the activation scale s = absmax / 7 (s > 0), with r the
// IEEE reciprocal of s.  |v / s| <= 7 (about), so v * r is within 2^-20 of
// the exact quotient and within 2^-19 of the IEEE quotient v / s; wherever
// v * r lies farther than 2^-19 from a half-integer both round to the same
// integer.  Nearer (or NaN, or an infinite r) the IEEE quotient decides, so
// every code equals rne(v / s) clamped, as the divide would give it.
__device__ __forceinline__ int quant_code_act(float v, float s, float r) {
  const float qa = v * r;
  float k = __builtin_rintf(qa);
  if (!(fabsf(qa - k) < 0.5f - 0x1p-19f)) k = __builtin_rintf(v / s);
  return (int)fminf(fmaxf(k, -8.0f), 7.0f);
}

// The 8-bit per-token code (W4A8 tier): rne(v / s) clamped to [-128, 127].
// |v / s| <= 127, so v * r is within 127 * 2^-23 < 2^-16 of the exact
// quotient and within 2^-15 of the IEEE quotient; farther than that from a
// half-integer both round alike, nearer the IEEE quotient decides.
__device__ __forceinline__ int quant_code_act8(float v, float s, float r) {
  const float qa = v * r;
  float k = __builtin_rintf(qa);
  if (!(fabsf(qa - k) < 0.5f - 0x1p-15f)) k = __builtin_rintf(v / s);
  return (int)fminf(fmaxf(k, -128.0f), 127.0f);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace qspec
