// Device-side helpers shared by the gfx950 kernels of the NVFP4 library.
//
// Formats (FlashInfer PR #3597, Description and review thread; FreeToken PR
// #737, Changes):
//   * e2m1 code: bit 3 sign, bits 2..0 magnitude index into {0, .5, 1, 1.5, 2,
//     3, 4, 6}; two codes per byte, the even-k element in the low nibble.
//   * block scale: one OCP FP8 E4M3 byte per 16 consecutive k (largest 448).
//   * dequantized value = e2m1(code) * E4M3(scale); every such product has at
//     most 6 significant bits and lies in [2^-10, 2688], so it is exact in
//     bf16 and in fp16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads.  The nontemporal form streams data that is read once (the
// weights of the decode linears) without keeping it in the caches.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld4_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// E4M3 byte (selected from a dword) -> f32, through gfx950's OCP E4M3FN convert.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

// Two e2m1 codes (byte SEL of word) -> two f32 values (low nibble first),
// exact.  The convert's scale operand only contributes its exponent, so 1.0
// leaves the values unscaled.
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, exact here
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));  // exact here
}

// Eight codes of one dword (k ascending: nibble 0 is the lowest k) times the
// block scale S -> eight bf16 values, as four packed dwords.
__device__ __forceinline__ void dequant8_bf16(uint32_t codes, float S, uint32_t out[4]) {
  const f32x2_t p0 = e2m1x2_to_f32<0>(codes);
  const f32x2_t p1 = e2m1x2_to_f32<1>(codes);
  const f32x2_t p2 = e2m1x2_to_f32<2>(codes);
  const f32x2_t p3 = e2m1x2_to_f32<3>(codes);
  out[0] = pack_bf16x2(p0.x * S, p0.y * S);
  out[1] = pack_bf16x2(p1.x * S, p1.y * S);
  out[2] = pack_bf16x2(p2.x * S, p2.y * S);
  out[3] = pack_bf16x2(p3.x * S, p3.y * S);
}

// Two e2m1 codes (byte SEL of word) -> two fp16 values (low nibble first),
// exact, by gfx950's packed fp4 -> fp16 convert (scale 1.0: unscaled).
template <int SEL>
__device__ __forceinline__ f16x2_t e2m1x2_to_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

// Same, to fp16: two codes per convert, then one packed fp16 multiply per pair
// applies S (both factors and the product are exact in fp16).
__device__ __forceinline__ void dequant8_f16(uint32_t codes, uint32_t S2 /* S as f16x2 */, uint32_t out[4]) {
  const f16x2_t s = __builtin_bit_cast(f16x2_t, S2);
  out[0] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<0>(codes) * s);
  out[1] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<1>(codes) * s);
  out[2] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<2>(codes) * s);
  out[3] = __builtin_bit_cast(uint32_t, e2m1x2_to_f16<3>(codes) * s);
}

__device__ __forceinline__ uint32_t f32_to_f16x2_splat(float s) {
  const uint32_t h = pack_f16x2_rtz(s, s);
  return h;
}

// SiLU(z) = z / (1 + e^-z) with the hardware base-2 exponential and
// reciprocal: a few ulp of relative error, far below the distances to the
// rounding boundaries of h that matter (an h within about 2^-14 of an NVFP4
// boundary may round either way against an fp64 reference anyway; a bf16 h
// keeps 8 bits).  Large |z| saturates correctly: e^-z = inf gives -0, e^-z =
// 0 gives z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace nvfp4
