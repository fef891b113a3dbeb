// W4A16 NVFP4 linear for decode-sized M (M <= 16) on gfx950.
//
// Computes out[m, n] = bf16(alpha * sum_k a[m, k] * e2m1(c[n, k]) * E4M3(s[n, k/16]))
// with fp32 accumulation (FlashInfer PR #3597, Description: out = (a @
// dequant(b, b_sf).T) * alpha), reading the canonical row-major [N, K/2] codes
// and [N, K/16] scales (FreeToken PR #737, Changes: one weight copy, no repack).
//
// Design (HBM-bound: every weight byte is read once; activations stay in L2):
//  * swap-AB bf16 MFMA 16x16x32: 16 weight rows on the MFMA's M side, up to 16
//    tokens on its N side (tokens >= M contribute zeros);
//  * k is permuted inside each 256-k step so that one lane's two dwordx4 code
//    loads (32 contiguous bytes = 64 k of one row) and its one scale dword are
//    exactly the A operands of 8 MFMAs; the activation operand uses the same
//    permutation (8 contiguous bf16 per lane per MFMA).  A row's 128 code bytes
//    of a step come from 4 lanes, so each wave instruction reads whole lines;
//  * dequant: fp4 -> f32 pair (hardware convert), times the E4M3 scale, packed
//    to bf16 -- exact, since e2m1 * E4M3 fits bf16;
//  * the K range is split across the waves of one workgroup, which then add
//    their partial 16x16 tiles through LDS in a fixed order (deterministic, no
//    workspace, one launch).  This fills the GPU at small N without a second
//    reduction kernel.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

// One wave: R row tiles (16 rows each) x S consecutive 256-k steps.  All of the
// wave's weight bytes (R*S*(32 B codes + 4 B scales) per lane) are requested
// before any arithmetic, so a CU holds tens of KB of HBM reads in flight; the
// activation operands of step s+1 are requested while step s computes.
template <int R, int S, int WMAX>
__global__ __launch_bounds__(64 * WMAX) void w4a16_kernel(const uint16_t* __restrict__ a, int64_t lda, int32_t M,
                                                          const uint8_t* __restrict__ wc,
                                                          const uint8_t* __restrict__ ws, int32_t N, int32_t K,
                                                          const float* __restrict__ alpha_p,
                                                          uint16_t* __restrict__ out, int64_t ldo) {
  extern __shared__ float red[];  // [waves][R][64][4]
  const int lane = int(threadIdx.x & 63);
  const int wave = int(threadIdx.x >> 6);
  const int nwaves = int(blockDim.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int32_t n_base = int32_t(blockIdx.x) * 16 * R;
  const int32_t steps = K / 256;
  const int32_t s0 = wave * S;
  const int64_t code_row = K / 2, scale_row = K / 16;

  uint4 cw[S][R][2];
  uint32_t sw[S][R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int32_t n = min(n_base + 16 * t + r, N - 1);
    const uint8_t* wrow = wc + int64_t(n) * code_row + 32 * q;
    const uint8_t* srow = ws + int64_t(n) * scale_row + 4 * q;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int32_t st = min(s0 + s, steps - 1);  // steps past the end are loaded but unused
      cw[s][t][0] = ld16_nt(wrow + 128 * int64_t(st));
      cw[s][t][1] = ld16_nt(wrow + 128 * int64_t(st) + 16);
      sw[s][t] = ld4_nt(srow + 16 * int64_t(st));
    }
  }
  const bool tok = r < M;
  const uint16_t* arow = a + int64_t(tok ? r : 0) * lda + 64 * q;

  f32x4_t acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 b[2][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[0][j] = make_uint4(0, 0, 0, 0);
  if (tok && s0 < steps) {
#pragma unroll
    for (int j = 0; j < 8; ++j) b[0][j] = ld16(arow + 256 * int64_t(s0) + 8 * j);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s0 + s >= steps) break;  // wave-uniform
    const int cur = s & 1;
    if (s + 1 < S) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[cur ^ 1][j] = make_uint4(0, 0, 0, 0);
      if (tok && s0 + s + 1 < steps) {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[cur ^ 1][j] = ld16(arow + 256 * int64_t(s0 + s + 1) + 8 * j);
      }
    }
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const uint32_t cwd[8] = {cw[s][t][0].x, cw[s][t][0].y, cw[s][t][0].z, cw[s][t][0].w,
                               cw[s][t][1].x, cw[s][t][1].y, cw[s][t][1].z, cw[s][t][1].w};
      const float Sg[4] = {e4m3_to_f32<0>(sw[s][t]), e4m3_to_f32<1>(sw[s][t]), e4m3_to_f32<2>(sw[s][t]),
                           e4m3_to_f32<3>(sw[s][t])};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t av[4];
        dequant8_bf16(cwd[j], Sg[j >> 1], av);
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(av[0], av[1], av[2], av[3]));
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b[cur][j]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < R; ++t)
    *reinterpret_cast<f32x4_t*>(&red[((wave * R + t) * 64 + lane) * 4]) = acc[t];
  __syncthreads();
  const float alpha = *alpha_p;
  for (int idx = int(threadIdx.x); idx < R * 64; idx += int(blockDim.x)) {
    const int t = idx >> 6, ln = idx & 63;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < nwaves; ++w) sum += *reinterpret_cast<const f32x4_t*>(&red[((w * R + t) * 64 + ln) * 4]);
    const int c = ln & 15, qq = ln >> 4;
    if (c < M) {
      uint16_t* orow = out + int64_t(c) * ldo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t n = n_base + 16 * t + 4 * qq + i;
        if (n < N) orow[n] = __builtin_bit_cast(uint16_t, (__bf16)(sum[i] * alpha));
      }
    }
  }
}

}  // namespace

// Largest waves-per-workgroup each steps-per-wave variant is compiled for.
constexpr int wmax_for(int S) { return S == 1 ? 16 : (S == 2 ? 16 : 8); }

W4A16Config w4a16_default_config(int64_t M, int64_t N, int64_t K) {
  W4A16Config c;
  const int64_t steps = K / 256;
  // steps per wave: keep a workgroup within 16 waves, two steps once K is long
  c.steps_per_wave = steps <= 8 ? 1 : (steps <= 32 ? 2 : 4);
  // row tiles per wave: as many as keep at least one workgroup per CU
  const int64_t tiles = (N + 15) / 16;
  c.row_tiles = 1;
  if (tiles / 4 >= 256 && c.steps_per_wave <= 2) c.row_tiles = 4;
  else if (tiles / 2 >= 256 || (M > 4 && tiles / 2 >= 128)) c.row_tiles = 2;
  if (c.row_tiles == 4 && c.steps_per_wave == 2) c.row_tiles = 2;  // register budget of the 16-wave variant
  return c;
}

bool w4a16_config_valid(const W4A16Config& c, int64_t K) {
  const int R = c.row_tiles, S = c.steps_per_wave;
  if (R != 1 && R != 2 && R != 4) return false;
  if (S != 1 && S != 2 && S != 4) return false;
  if (R * S > 4 && !(R == 2 && S == 4)) return false;
  const int64_t steps = K / 256;
  const int64_t waves = (steps + S - 1) / S;
  return waves >= 1 && waves <= wmax_for(S);
}

namespace {
template <int R, int S>
void launch_rs(dim3 grid, int waves, size_t lds, hipStream_t stream, const uint16_t* A, int64_t lda, int32_t M,
               const uint8_t* WC, const uint8_t* WS, int32_t N, int32_t K, const float* alpha, uint16_t* O,
               int64_t ldo) {
  hipLaunchKernelGGL((w4a16_kernel<R, S, wmax_for(S)>), grid, dim3(64 * waves), lds, stream, A, lda, M, WC, WS, N, K,
                     alpha, O, ldo);
}
}  // namespace

hipError_t launch_w4a16(const void* a, int64_t M, int64_t lda, const void* w_codes, const void* w_scales,
                        int64_t N, int64_t K, const float* alpha, void* out, int64_t ldo,
                        const W4A16Config& cfg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t steps = K / 256;
  const int S = cfg.steps_per_wave, R = cfg.row_tiles;
  const int waves = int((steps + S - 1) / S);
  const dim3 grid(uint32_t((N + 16 * R - 1) / (16 * R)));
  const size_t lds = size_t(waves) * R * 64 * 4 * sizeof(float);
  const auto* A = static_cast<const uint16_t*>(a);
  const auto* WC = static_cast<const uint8_t*>(w_codes);
  const auto* WS = static_cast<const uint8_t*>(w_scales);
  auto* O = static_cast<uint16_t*>(out);
  const int32_t m = int32_t(M), n = int32_t(N), k = int32_t(K);
#define NVFP4_W4A16_CASE(RR, SS) \
  if (R == RR && S == SS) launch_rs<RR, SS>(grid, waves, lds, stream, A, lda, m, WC, WS, n, k, alpha, O, ldo);
  NVFP4_W4A16_CASE(1, 1)
  NVFP4_W4A16_CASE(1, 2)
  NVFP4_W4A16_CASE(1, 4)
  NVFP4_W4A16_CASE(2, 1)
  NVFP4_W4A16_CASE(2, 2)
  NVFP4_W4A16_CASE(2, 4)
  NVFP4_W4A16_CASE(4, 1)
#undef NVFP4_W4A16_CASE
  return hipGetLastError();
}

}  // namespace nvfp4
