// NVFP4 quantization of bf16 rows on gfx950, plus the calibration helpers
// (per-tensor global scale and alpha).
//
// What is computed (FlashInfer PR #3597, Description and API example; FreeToken
// PR #737, Changes, where the activation quantizer works on blocks of a row
// rather than whole rows):
//   for every 16 consecutive elements of a row:
//     amax   = max |x|
//     scale  = the E4M3 byte nearest to amax*g/6 (ties to even, saturating 448)
//     code_i = sign(x_i) | the e2m1 index nearest to |x_i|*g/S (ties to even,
//              saturating 6), S = value of the scale byte
//   two codes per byte, the even-k element in the low nibble; scales row-major.
// Both roundings decide on the exact real values amax*g/6 and |x|*g/S.
//
// Mapping: one lane per 16-element block; a wave covers 64 consecutive blocks
// (2 KB of contiguous bf16 through dwordx4 loads) of 2 rows, a workgroup 8
// rows.  The block max is an integer max over bf16 magnitude bits.  The loads
// are ordinary (cached) ones: on the prefill activations (M = 8192, K = 5120)
// 2 rows per wave and cached loads took a call from 32.7 to 29.7 us on cold
// inputs and from 25.8 to 20.0 us on an input the caches still hold (4 rows
// per wave with nontemporal loads before; bit-identical).
//
// Rounding of the codes: the fast path forms w = x * fl(g/S) and lets the
// hardware f32 -> e2m1 convert round it (nearest, ties to even, saturating,
// sign kept -- checked against the oracle).  w differs from the exact real
// value by at most two fp32 ulps, so the result can only differ when w lies
// within a few ulps of a rounding threshold (0.25, 0.75, 1.25, 1.75, 2.5, 3.5
// or 5 -- all with their low 21 mantissa bits zero).  A lane that sees such a
// w recomputes its block by exact comparisons: the sign of fma(|x|, g, -T*S)
// is the sign of the exact |x|*g - T*S (T*S is exact in fp32).
#include "device.hpp"
#include "kernels.hpp"
#include "quant_exact.hpp"

namespace nvfp4 {

namespace {

template <int SEL>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t acc, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, SEL);
}

// Per-call tables, indexed by the scale byte s = 0..126, built once per
// workgroup in LDS (exact: the same operations the per-block code would do):
//   val[s]  = E4M3 value of s
//   gs[s]   = fl(g / val[s]) (0 for s = 0)
//   mid6[s] = 3 * (val[s-1] + val[s]) = 6 x the midpoint below s (s >= 1)
struct ScaleTables {
  float val[128], gs[128], mid6[128];
};

// The E4M3 byte nearest to the exact amax*g/6: the same decision as
// scale_byte(), with the values and midpoints read from the tables.
__device__ __forceinline__ uint32_t scale_byte_lut(float amax, float g, const ScaleTables& T) {
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
    const float d = __builtin_fmaf(amax, g, -T.mid6[s]);
    if (d < 0.0f || (d == 0.0f && ((s - 1) & 1u) == 0)) s -= 1;
  }
  if (s < 126) {
    const float d = __builtin_fmaf(amax, g, -T.mid6[s + 1]);
    if (d > 0.0f || (d == 0.0f && ((s + 1) & 1u) == 0)) s += 1;
  }
  return s;
}

// Codes and scale of one 16-element block (eight bf16 pairs in d).
// SMALL_G: g has at most 8 significant bits (its low 16 mantissa bits are
// zero).  Then x*g is exact in fp32 (8 + 8 bits), and x*g/S is either exactly
// a value of at most 3 significant bits (a rounding threshold, or a code) or
// at least about 2^-16 of itself away from every such value, since x*g - T*S
// is then a nonzero multiple of the quantum of x*g.  w = x*fl(g/S) lies
// within 2^-22 of x*g/S, so the convert of w rounds the right way except on
// an exact tie: there w is snapped to its nearest 2-mantissa-bit value tn
// when x*g == tn*S (both products exact), and the convert's ties-to-even
// takes the even code.  No exact fallback is needed on this path.
template <bool SMALL_G>
__device__ __forceinline__ void quantize_block(const uint32_t (&d)[8], float g, const ScaleTables& T, uint32_t& c0,
                                               uint32_t& c1, uint32_t& s) {
  uint32_t mbits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mbits = max(mbits, max(d[i] & 0x7FFFu, (d[i] >> 16) & 0x7FFFu));
  const float amax = bf16_bits_to_f32(mbits);
  s = scale_byte_lut(amax, g, T);
  const float G = T.gs[s];

  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(d[i] << 16);
    x[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
  }
  c0 = 0;
  c1 = 0;
  float w[16];
  bool near = false;
  if (SMALL_G) {
    const float S = T.val[s];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[i] = x[i] * G;
      const float tn = __uint_as_float((__float_as_uint(w[i]) + 0x100000u) & 0xFFE00000u);
      w[i] = x[i] * g == tn * S ? tn : w[i];
    }
  } else {
    // near_threshold() for all 16 at once: (bits + 4) << 11 keeps the low 21
    // bits plus 4, scaled to the top of the word; w is within 4 ulps of a
    // value whose low 21 bits are zero iff that is below 9 << 11
    uint32_t dmin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[i] = x[i] * G;
      dmin = min(dmin, (__float_as_uint(w[i]) << 11) + (4u << 11));
    }
    near = dmin < (9u << 11);
  }
  c0 = cvt_pair<0>(c0, w[0], w[1]);
  c0 = cvt_pair<1>(c0, w[2], w[3]);
  c0 = cvt_pair<2>(c0, w[4], w[5]);
  c0 = cvt_pair<3>(c0, w[6], w[7]);
  c1 = cvt_pair<0>(c1, w[8], w[9]);
  c1 = cvt_pair<1>(c1, w[10], w[11]);
  c1 = cvt_pair<2>(c1, w[12], w[13]);
  c1 = cvt_pair<3>(c1, w[14], w[15]);

  if (!SMALL_G && near && s != 0) {
    const float S = T.val[s];
    c0 = 0;
    c1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0 |= exact_code(x[i], g, S) << (4 * i);
      c1 |= exact_code(x[8 + i], g, S) << (4 * i);
    }
  }
}

// A wave takes kRowsPerWave rows of one 64-block column range; all their
// loads are issued before the tables are built and the first block is
// computed (rows past the last re-read it and are not stored).  Two rows per
// wave suit large batches; a small batch is latency-bound, and one row per
// wave halves each wave's serial work (next to the few-rows GEMM on N =
// 62080, K = 5120: 6.0 -> 4.1 us at M = 64, 4.2 -> 2.7 us at M = 128; at
// M = 8192 two rows stay faster).
constexpr int64_t kQuantizeOneRowMax = 256;  // rows up to which a wave takes one row

template <int kRowsPerWave>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                       int32_t rows, int32_t blocks_per_row,
                                                       const float* __restrict__ g_ptr,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int32_t swz_cols,
                                                       int32_t rows_pad) {
  __shared__ ScaleTables T;
  const int32_t j = int32_t(blockIdx.x) * 64 + int32_t(threadIdx.x & 63);
  const int32_t row0 = (int32_t(blockIdx.y) * 4 + int32_t(threadIdx.x >> 6)) * kRowsPerWave;
  const bool active = j < blocks_per_row && row0 < rows;
  uint4 v[kRowsPerWave][2];
  if (active) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const uint16_t* src = a + int64_t(min(row0 + r, rows - 1)) * lda + int64_t(j) * 16;
      v[r][0] = ld16(src);
      v[r][1] = ld16(src + 8);
    }
  }
  const float g = *g_ptr;
  if (threadIdx.x < 128) {
    const uint32_t sb = min(uint32_t(threadIdx.x), 126u);
    const float val = e4m3_pos_value(sb);
    T.val[threadIdx.x] = val;
    T.gs[threadIdx.x] = sb == 0 ? 0.0f : g / val;
    T.mid6[threadIdx.x] = sb == 0 ? 0.0f : 3.0f * (e4m3_pos_value(sb - 1) + val);
  }
  __syncthreads();
  if (!active) {
    // swizzled scales: the padding rows (up to a multiple of 128) and columns
    // (up to a multiple of 4) are zero
    if (swz_cols > 0 && j < swz_cols)
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int32_t row = row0 + r;
        if (row < rows_pad && (row >= rows || j >= blocks_per_row))
          scales[swizzled_scale_offset(row, j, swz_cols)] = 0;
      }
    return;
  }
  const int32_t half_k = blocks_per_row * 8;
  // g with at most 8 significant bits: the exact path of quantize_block<true>
  const bool small_g = (__float_as_uint(g) & 0xFFFFu) == 0;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const uint32_t d[8] = {v[r][0].x, v[r][0].y, v[r][0].z, v[r][0].w, v[r][1].x, v[r][1].y, v[r][1].z, v[r][1].w};
    uint32_t c0, c1, s;
    if (small_g)
      quantize_block<true>(d, g, T, c0, c1, s);
    else
      quantize_block<false>(d, g, T, c0, c1, s);
    const int32_t row = row0 + r;
    if (row < rows) {
      *reinterpret_cast<uint2*>(codes + int64_t(row) * half_k + int64_t(j) * 8) = make_uint2(c0, c1);
      scales[swz_cols > 0 ? swizzled_scale_offset(row, j, swz_cols) : int64_t(row) * blocks_per_row + j] =
          uint8_t(s);
    } else if (swz_cols > 0 && row < rows_pad) {
      scales[swizzled_scale_offset(row, j, swz_cols)] = 0;
    }
  }
}

// ---------------------------------------------------------------- calibration

__global__ void set_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

// max |x| over a bf16 matrix, as bf16 magnitude bits, into *out (atomic max).
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                   int64_t ld, uint32_t* __restrict__ out) {
  const int64_t chunks = cols / 8;
  const int64_t total = rows * chunks;
  uint32_t m = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / chunks, c = i - r * chunks;
    const uint4 v = *reinterpret_cast<const uint4*>(x + r * ld + c * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(d[k] & 0x7FFFu, (d[k] >> 16) & 0x7FFFu));
  }
  for (int o = 32; o > 0; o >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), o, 64)));
  if ((threadIdx.x & 63) == 0) atomicMax(out, m);
}

// g = fp32(448 * 6 / amax) with IEEE fp32 division (0 for an all-zero tensor).
__global__ void global_from_amax_kernel(uint32_t* inout) {
  const float amax = bf16_bits_to_f32(*inout);
  const float g = amax > 0.0f ? 2688.0f / amax : 0.0f;
  *reinterpret_cast<float*>(inout) = g;
}

// alpha = fp32(1 / (g_w * g_a)) with the product and quotient in double; g_a
// may be null (W4A16 alpha = fp32(1 / g_w)).
__global__ void alpha_kernel(const float* gw, const float* ga, float* alpha) {
  const double den = ga ? double(*gw) * double(*ga) : double(*gw);
  *alpha = float(1.0 / den);
}

}  // namespace

hipError_t launch_quantize(const void* a, int64_t M, int64_t K, int64_t lda, const float* g, void* codes,
                           void* scales, hipStream_t stream, int64_t swz_cols) {
  if (M == 0) return hipSuccess;
  const int32_t bpr = int32_t(K / 16);
  const int64_t rows = swz_cols > 0 ? (M + 127) / 128 * 128 : M;  // the grid covers the padding rows
  const dim3 gx((bpr + 63) / 64, 1);
  if (rows <= kQuantizeOneRowMax) {
    const dim3 grid(gx.x, uint32_t((rows + 3) / 4));
    hipLaunchKernelGGL(quantize_kernel<1>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(a), lda,
                       int32_t(M), bpr, g, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                       int32_t(swz_cols), int32_t(rows));
  } else {
    const dim3 grid(gx.x, uint32_t((rows + 7) / 8));
    hipLaunchKernelGGL(quantize_kernel<2>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(a), lda,
                       int32_t(M), bpr, g, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                       int32_t(swz_cols), int32_t(rows));
  }
  return hipGetLastError();
}

hipError_t launch_global_scale(const void* x, int64_t rows, int64_t cols, int64_t ld, float* g_out,
                               hipStream_t stream) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(g_out);
  hipLaunchKernelGGL(set_u32_kernel, dim3(1), dim3(1), 0, stream, bits, 0u);
  const int64_t total = rows * (cols / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), rows, cols, ld, bits);
  hipLaunchKernelGGL(global_from_amax_kernel, dim3(1), dim3(1), 0, stream, bits);
  return hipGetLastError();
}

hipError_t launch_alpha(const float* g_w, const float* g_a, float* alpha, hipStream_t stream) {
  hipLaunchKernelGGL(alpha_kernel, dim3(1), dim3(1), 0, stream, g_w, g_a, alpha);
  return hipGetLastError();
}

}  // namespace nvfp4
