// W4A4 NVFP4 linear (prefill-sized M) on gfx950.
//
// Computes out[m, n] = bf16(alpha * sum_k deq(A)[m, k] * deq(W)[n, k]) with
// alpha = 1 / (g_w * g_a), on NVFP4 activations (from the quantize kernel) and
// the same prepared (tiled) weight as the W4A16 path (FreeToken PR #737,
// Changes: both linears use one weight copy).
//
// Arithmetic: every dequantized value e2m1 * E4M3 is exact in fp16, so the
// tile product runs on the fp16 MFMA with exact operands and fp32
// accumulation.  (gfx950's fp4 MFMA applies power-of-two block scales per 32
// k, which cannot carry NVFP4's per-16 E4M3 scales exactly.)  Dequant is one
// hardware fp4 -> f32 pair convert, one f32 -> f16 pack and one packed fp16
// multiply per two elements, done once per workgroup tile into LDS.
//
// Tile: 128 (n) x 128 (m) x 64 (k); four waves, each 64 x 64 of 16x16x32 fp16
// MFMAs with the weight on the MFMA's row side so a lane ends with 4
// consecutive n of one m.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

constexpr int BN = 128, BM = 128, BK = 64;
constexpr int PITCH = BK + 8;  // fp16 per LDS row; the pad staggers rows across banks

// Each of the 256 threads loads 16 code bytes (32 k) of one row of the tile
// plus the scale dword of that row, and later writes the 32 dequantized fp16.
struct Stage {
  uint4 codes;
  uint32_t scales;
};

__device__ __forceinline__ Stage load_stage(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                            int64_t row, int64_t K, int kb, int half) {
  Stage s;
  s.codes = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + int64_t(kb) * (BK / 2) + 16 * half);
  s.scales = *reinterpret_cast<const uint32_t*>(scales + row * (K / 16) + int64_t(kb) * (BK / 16));
  return s;
}

// Weight stage from the tiled layout: row n of the weight, 64-k block kb, the
// 32 k of half `half` (scale groups 4p + q for q = 2*half, 2*half + 1 of step
// kb/4, p = kb % 4).  Unit (t, s) holds, for lane r + 16q, the codes of groups
// q, 4+q at byte 16*lane, of groups 8+q, 12+q at 1024 + 16*lane, and the four
// scale bytes at 2048 + 4*lane.
__device__ __forceinline__ Stage load_w_stage(const uint8_t* __restrict__ wt, int64_t n, int32_t steps, int kb,
                                              int half) {
  const int64_t t = n >> 4, r = n & 15;
  const int s = kb >> 2, p = kb & 3;
  const uint8_t* u = wt + (t * steps + s) * 2304;
  const int64_t l0 = r + 16 * (2 * half), l1 = l0 + 16;
  const uint2 a = *reinterpret_cast<const uint2*>(u + 1024 * (p >> 1) + 16 * l0 + 8 * (p & 1));
  const uint2 b = *reinterpret_cast<const uint2*>(u + 1024 * (p >> 1) + 16 * l1 + 8 * (p & 1));
  Stage st;
  st.codes = make_uint4(a.x, a.y, b.x, b.y);
  st.scales = (uint32_t(u[2048 + 4 * l0 + p]) | (uint32_t(u[2048 + 4 * l1 + p]) << 8)) << (16 * half);
  return st;
}

__device__ __forceinline__ void store_stage(const Stage& s, int half, _Float16* dst) {
  // this thread's 32 k use scale groups 2*half and 2*half + 1
  const uint32_t sb = s.scales >> (16 * half);
  const uint32_t S0 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(sb, 0));
  const uint32_t S1 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(sb, 1));
  uint32_t v[16];
  dequant8_f16(s.codes.x, S0, v + 0);
  dequant8_f16(s.codes.y, S0, v + 4);
  dequant8_f16(s.codes.z, S1, v + 8);
  dequant8_f16(s.codes.w, S1, v + 12);
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(v[0], v[1], v[2], v[3]);
  d[1] = make_uint4(v[4], v[5], v[6], v[7]);
  d[2] = make_uint4(v[8], v[9], v[10], v[11]);
  d[3] = make_uint4(v[12], v[13], v[14], v[15]);
}

__global__ __launch_bounds__(256) void w4a4_kernel(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                                   int32_t M, const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                   const float* __restrict__ alpha_p, uint16_t* __restrict__ out,
                                                   int64_t ldo) {
  __shared__ __attribute__((aligned(16))) _Float16 lw[BN * PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 la[BM * PITCH];
  const int tid = int(threadIdx.x);
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int i16 = lane & 15, q = lane >> 4;
  const int32_t n0 = int32_t(blockIdx.x) * BN, m0 = int32_t(blockIdx.y) * BM;

  // loader role: row tid/2 of both tiles, 32 k half (tid & 1)
  const int lrow = tid >> 1, half = tid & 1;
  const int32_t steps = K / 256;
  const int64_t wrow = min(n0 + lrow, (N + 15) / 16 * 16 - 1);
  const int64_t arow = min(m0 + lrow, M - 1);
  _Float16* lw_dst = lw + lrow * PITCH + 32 * half;
  _Float16* la_dst = la + lrow * PITCH + 32 * half;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  Stage sw = load_w_stage(wt, wrow, steps, 0, half);
  Stage sa = load_stage(ac, as, arow, K, 0, half);
  for (int kb = 0; kb < nk; ++kb) {
    __syncthreads();
    store_stage(sw, half, lw_dst);
    store_stage(sa, half, la_dst);
    __syncthreads();
    if (kb + 1 < nk) {
      sw = load_w_stage(wt, wrow, steps, kb + 1, half);
      sa = load_stage(ac, as, arow, K, kb + 1, half);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      f16x8_t A[4], B[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        A[t] = *reinterpret_cast<const f16x8_t*>(lw + (wn * 64 + 16 * t + i16) * PITCH + 32 * kk + 8 * q);
        B[t] = *reinterpret_cast<const f16x8_t*>(la + (wm * 64 + 16 * t + i16) * PITCH + 32 * kk + 8 * q);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[i], B[j], acc[i][j], 0, 0, 0);
    }
  }

  const float alpha = *alpha_p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int32_t m = m0 + wm * 64 + 16 * j + i16;
      if (m >= M) continue;
      uint16_t* orow = out + int64_t(m) * ldo;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int32_t n = n0 + wn * 64 + 16 * i + 4 * q + v;
        if (n < N) orow[n] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][j][v] * alpha));
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid(uint32_t((N + BN - 1) / BN), uint32_t((M + BM - 1) / BM));
  hipLaunchKernelGGL(w4a4_kernel, grid, dim3(256), 0, stream, static_cast<const uint8_t*>(a_codes),
                     static_cast<const uint8_t*>(a_scales), int32_t(M), static_cast<const uint8_t*>(w_tiled),
                     int32_t(N), int32_t(K), alpha,
                     static_cast<uint16_t*>(out), ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
