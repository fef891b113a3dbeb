// W4A4 NVFP4 linear (prefill-sized M) on gfx950.
//
// Computes out[m, n] = bf16(alpha * sum_k deq(A)[m, k] * deq(W)[n, k]) with
// alpha = 1 / (g_w * g_a), on NVFP4 activations (from the quantize kernel) and
// the same prepared (tiled) weight as the W4A16 path (FreeToken PR #737,
// Changes: prefill runs W4A4 GEMMs on NVFP4 activations, one weight copy).
// The main loop is gemm::mainloop (256 weight rows x 256 activation rows per
// workgroup, fp16 MFMA on exactly dequantized operands).
#include "gemm_w4a4.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(gemm::kThreads) void w4a4_kernel(const uint8_t* __restrict__ ac,
                                                              const uint8_t* __restrict__ as, int32_t M,
                                                              const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                              const float* __restrict__ alpha_p,
                                                              uint16_t* __restrict__ out, int64_t ldo, int vec_store) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int32_t tiles = (N + 15) / 16;
  int32_t nblk, mblk;
  if (!gemm::xcd_tile(int32_t(blockIdx.x), (N + gemm::BN - 1) / gemm::BN, (M + gemm::BM - 1) / gemm::BM, nblk, mblk))
    return;
  const int32_t tb = nblk * (gemm::BN / 16);  // first weight tile of the workgroup
  const int32_t m0 = mblk * gemm::BM;
  gemm::Acc acc;
  gemm::mainloop(
      acc, lds, ac, as, [&](int i) { return int64_t(min(m0 + i, M - 1)); }, wt,
      [&](int lt) { return int64_t(min(tb + lt, tiles - 1)); }, [&](int t) { return 128 * wn + 32 * t; }, K);

  // register i of tile (t, u): weight row 16*tb + 128*wn + 32t + 8(i/4) + 4h + i%4,
  // activation row m0 + 64*wm + 32u + (lane % 32)
  const float alpha = *alpha_p;
  if (vec_store) {
    gemm::store_tile_lds(
        lds, [&](int t, int u, int i) { return acc.v[t][u][i] * alpha; }, out, ldo, m0, M, 16 * tb, N);
    return;
  }
  const int h = lane >> 5;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int32_t m = m0 + wm * 64 + 32 * u + (lane & 31);
    if (m >= M) continue;
    uint16_t* orow = out + int64_t(m) * ldo;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int32_t n = 16 * tb + 128 * wn + 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
        if (n < N) orow[n] = __builtin_bit_cast(uint16_t, (__bf16)(acc.v[t][u][i] * alpha));
      }
    }
  }
}

}  // namespace

hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid(uint32_t(gemm::xcd_grid(int32_t((N + gemm::BN - 1) / gemm::BN) * int32_t((M + gemm::BM - 1) / gemm::BM))));
  // whole 16-byte output pieces when the rows are 16-byte aligned
  const int vec_store = (reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * 2) % 16 == 0) ? 1 : 0;
  hipLaunchKernelGGL(w4a4_kernel, grid, dim3(gemm::kThreads), 0, stream, static_cast<const uint8_t*>(a_codes),
                     static_cast<const uint8_t*>(a_scales), int32_t(M), static_cast<const uint8_t*>(w_tiled),
                     int32_t(N), int32_t(K), alpha, static_cast<uint16_t*>(out), ldo, vec_store);
  return hipGetLastError();
}

}  // namespace nvfp4
