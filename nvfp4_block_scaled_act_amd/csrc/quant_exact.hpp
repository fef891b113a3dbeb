// Exact NVFP4 rounding decisions on fp32 inputs, shared by the activation
// quantizer and the MoE gate_up epilogue (which quantizes its fp32 h).
//
// Both roundings decide on exact real values (FlashInfer PR #3597,
// Description: scale = E4M3(amax * g / 6), code = e2m1(x * g / S)): a fused
// multiply-add forms |x|*g - T*S with a single rounding, so its sign is the
// sign of the exact difference whenever T*S is exact in fp32 (T and S have at
// most 4 significant bits, their products and the E4M3 midpoints times 6 at
// most 7).
#pragma once

#include "device.hpp"

namespace nvfp4 {

// Value of a non-negative E4M3 byte 0x00..0x7E (exact in fp32).
__device__ __forceinline__ float e4m3_pos_value(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e == 0 ? float(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// The E4M3 byte nearest to the exact amax*g/6.  An fp32 estimate picks a
// candidate that is at most one byte off; the two neighbouring midpoints are
// then compared exactly (6*midpoint has at most 7 significant bits).
__device__ __forceinline__ uint32_t scale_byte(float amax, float g) {
  const float t = amax * g * (1.0f / 6.0f);
  uint32_t s;
  if (!(t < 464.0f)) {
    s = 126;
  } else if (t < 0x1p-6f) {
    s = uint32_t(__builtin_rintf(t * 512.0f));  // subnormal range, 0..8
  } else {
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u);  // round the fp32 mantissa to 3 bits
    s = min(((u >> 23) - 120u) * 8u + ((u >> 20) & 7u), 126u);
  }
  if (s > 0) {
    const float d = __builtin_fmaf(amax, g, -3.0f * (e4m3_pos_value(s - 1) + e4m3_pos_value(s)));
    if (d < 0.0f || (d == 0.0f && ((s - 1) & 1u) == 0)) s -= 1;
  }
  if (s < 126) {
    const float d = __builtin_fmaf(amax, g, -3.0f * (e4m3_pos_value(s) + e4m3_pos_value(s + 1)));
    if (d > 0.0f || (d == 0.0f && ((s + 1) & 1u) == 0)) s += 1;
  }
  return s;
}

// Exact e2m1 code of x under scale S (S > 0): a three-level search over the
// thresholds 0.25..5 (x S).  Thresholds below odd indices round down on a tie
// (>), the others up (>=), which is ties-to-even.
__device__ __forceinline__ uint32_t exact_code(float x, float g, float S) {
  const float ax = __builtin_fabsf(x);
  const bool c2 = __builtin_fmaf(ax, g, -1.75f * S) >= 0.0f;
  const bool c1 = __builtin_fmaf(ax, g, -(c2 ? 3.5f : 0.75f) * S) >= 0.0f;
  const float t0 = c2 ? (c1 ? 5.0f : 2.5f) : (c1 ? 1.25f : 0.25f);
  const bool c0 = __builtin_fmaf(ax, g, -t0 * S) > 0.0f;
  const uint32_t mag = (c2 ? 4u : 0u) | (c1 ? 2u : 0u) | (c0 ? 1u : 0u);
  return ((__float_as_uint(x) >> 28) & 8u) | mag;
}

__device__ __forceinline__ bool near_threshold(float w) {
  return ((__float_as_uint(w) + 4u) & 0x1FFFFFu) <= 8u;
}

// Scale byte and codes of one block of 16 fp32 values by exact comparisons
// only: c0 holds the codes of x[0..7], c1 of x[8..15] (element 0 in the low
// nibble).  A zero scale gives zero magnitudes with the signs of x.
__device__ __forceinline__ uint32_t quantize16_exact(const float x[16], float g, uint32_t& c0, uint32_t& c1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  const uint32_t s = scale_byte(amax, g);
  const float S = e4m3_pos_value(s);
  c0 = 0;
  c1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c0 |= (s == 0 ? (__float_as_uint(x[i]) >> 28) & 8u : exact_code(x[i], g, S)) << (4 * i);
    c1 |= (s == 0 ? (__float_as_uint(x[8 + i]) >> 28) & 8u : exact_code(x[8 + i], g, S)) << (4 * i);
  }
  return s;
}

// Same result as quantize16_exact() with the codes from the hardware
// f32 -> e2m1 convert (round to nearest even, saturating, sign kept) of
// w = x * fl(g/S), which lies within two fp32 ulps of the exact x*g/S; the
// exact comparisons run only for a block holding a w within 4 ulps of a
// rounding threshold (0.25 .. 5, all with their low 21 mantissa bits zero).
__device__ __forceinline__ uint32_t quantize16_fast(const float x[16], float g, uint32_t& c0, uint32_t& c1) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  const uint32_t s = scale_byte(amax, g);
  const float S = e4m3_pos_value(s);
  const float G = s == 0 ? 0.0f : g / S;
  float w[16];
  uint32_t dmin = 0xFFFFFFFFu;  // (bits + 4) << 11: below 9 << 11 iff within 4 ulps of a threshold
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w[i] = x[i] * G;
    dmin = min(dmin, (__float_as_uint(w[i]) << 11) + (4u << 11));
  }
  c0 = 0;
  c1 = 0;
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, w[0], w[1], 1.0f, 0);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, w[2], w[3], 1.0f, 1);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, w[4], w[5], 1.0f, 2);
  c0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c0, w[6], w[7], 1.0f, 3);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, w[8], w[9], 1.0f, 0);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, w[10], w[11], 1.0f, 1);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, w[12], w[13], 1.0f, 2);
  c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c1, w[14], w[15], 1.0f, 3);
  if (dmin < (9u << 11) && s != 0) {
    c0 = 0;
    c1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0 |= exact_code(x[i], g, S) << (4 * i);
      c1 |= exact_code(x[8 + i], g, S) << (4 * i);
    }
  }
  return s;
}

}  // namespace nvfp4
