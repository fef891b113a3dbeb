// W4A4 NVFP4 linear (prefill-sized M) on gfx950.
//
// Computes out[m, n] = bf16(alpha * sum_k deq(A)[m, k] * deq(W)[n, k]) with
// alpha = 1 / (g_w * g_a), on NVFP4 activations (from the quantize kernel) and
// the same prepared (tiled) weight as the W4A16 path (FreeToken PR #737,
// Changes: prefill runs W4A4 GEMMs on NVFP4 activations, one weight copy).
// The main loop is gemm::mainloop (256 weight rows x 256 activation rows per
// workgroup, fp16 MFMA on exactly dequantized operands).
//
// One workgroup fills a CU (LDS), so the tiles run in rounds of one per CU.
// When the last round would be at most half full, its tiles are split into
// two 128-row halves each, which take about half as long.
#include "gemm_w4a4.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace nvfp4 {

namespace {

// Output of one tile: out[m][n] = bf16(chunk values) for activation rows m0..
// and weight rows 16*tb.., chunk(t, u, g) = the values of accumulator
// registers 4g .. 4g+3 of wave tile (t, u) (register i: weight row 16*tb +
// 128*wn + 32t + 8(i/4) + 4h + i%4, activation row m0 + (BMT/4)*wm + 32u +
// (lane % 32)).
template <int BMT, typename Chunk>
__device__ __forceinline__ void w4a4_store(_Float16* __restrict__ lds, Chunk chunk, int32_t M, int32_t N,
                                           uint16_t* __restrict__ out, int64_t ldo, int vec_store, int32_t tb,
                                           int32_t m0) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  if (vec_store) {
    gemm::store_tile_lds<BMT>(lds, chunk, out, ldo, m0, M, 16 * tb, N);
    return;
  }
  const int h = lane >> 5;
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u) {
    const int32_t m = m0 + wm * (BMT / 4) + 32 * u + (lane & 31);
    if (m >= M) continue;
    uint16_t* orow = out + int64_t(m) * ldo;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = chunk(t, u, g);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t n = 16 * tb + 128 * wn + 32 * t + 8 * g + 4 * h + e;
          if (n >= N) continue;
          orow[n] = __builtin_bit_cast(uint16_t, (__bf16)vv[e]);
        }
      }
    }
  }
}

template <int BMT>
__device__ __forceinline__ float4 acc_chunk(const gemm::AccT<BMT>& acc, int t, int u, int g, float alpha) {
  return make_float4(acc.v[t][u][4 * g] * alpha, acc.v[t][u][4 * g + 1] * alpha, acc.v[t][u][4 * g + 2] * alpha,
                     acc.v[t][u][4 * g + 3] * alpha);
}

template <int BMT>
__device__ __forceinline__ void w4a4_tile(_Float16* __restrict__ lds, const uint8_t* __restrict__ ac,
                                          const uint8_t* __restrict__ as, int32_t M, const uint8_t* __restrict__ wt,
                                          int32_t N, int32_t K, float alpha, uint16_t* __restrict__ out, int64_t ldo,
                                          int vec_store, int32_t nblk, int32_t m0) {
  const int32_t tb = nblk * (gemm::BN / 16);  // first weight tile of the workgroup
  const int wn = int(threadIdx.x >> 6) & 1;
  const int32_t tiles = (N + 15) / 16;
  gemm::AccT<BMT> acc;
  gemm::mainloop<false, BMT>(
      acc, lds, ac, as, [&](int i) { return int64_t(min(m0 + i, M - 1)); }, wt,
      [&](int lt) { return int64_t(min(tb + lt, tiles - 1)); }, [&](int t) { return 128 * wn + 32 * t; }, K);
  w4a4_store<BMT>(
      lds, [&](int t, int u, int g) { return acc_chunk<BMT>(acc, t, u, g, alpha); }, M, N, out, ldo, vec_store, tb,
      m0);
}

// Workgroups [0, grid_big) run the first n_big tiles of the grouped order as
// 256-row tiles (XCD-aware); the rest run the remaining tiles as 128-row halves.
__global__ __launch_bounds__(gemm::kThreads) void w4a4_kernel(const uint8_t* __restrict__ ac,
                                                              const uint8_t* __restrict__ as, int32_t M,
                                                              const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                              const float* __restrict__ alpha_p,
                                                              uint16_t* __restrict__ out, int64_t ldo, int vec_store,
                                                              int32_t n_big, int32_t grid_big) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  const int32_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  const float alpha = *alpha_p;
  int32_t nblk, mblk;
  const int32_t id = int32_t(blockIdx.x);
  if (id < grid_big) {
    if (!gemm::xcd_tile(id, nt, mt, n_big, nblk, mblk)) return;
    w4a4_tile<gemm::BM>(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, nblk, mblk * gemm::BM);
  } else {
    const int32_t j = id - grid_big;
    gemm::grouped_tile(n_big + j / 2, nt, mt, nblk, mblk);
    const int32_t m0 = mblk * gemm::BM + (gemm::BM / 2) * (j & 1);
    if (m0 >= M) return;
    w4a4_tile<gemm::BM / 2>(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, nblk, m0);
  }
}

}  // namespace

hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t total = ((N + gemm::BN - 1) / gemm::BN) * ((M + gemm::BM - 1) / gemm::BM);
  const int64_t cus = device_cu_count();
  const int64_t rest = total % cus;
  // split the last round into halves when it is at most half full
  const int64_t n_big = (total > cus && rest > 0 && 2 * rest <= cus) ? total - rest : total;
  const int64_t grid_big = gemm::xcd_grid(int32_t(n_big));
  const int64_t grid = grid_big + 2 * (total - n_big);
  // whole 16-byte output pieces when the rows are 16-byte aligned
  const int vec_store = (reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * 2) % 16 == 0) ? 1 : 0;
  hipLaunchKernelGGL(w4a4_kernel, dim3(uint32_t(grid)), dim3(gemm::kThreads), 0, stream,
                     static_cast<const uint8_t*>(a_codes), static_cast<const uint8_t*>(a_scales), int32_t(M),
                     static_cast<const uint8_t*>(w_tiled), int32_t(N), int32_t(K), alpha, static_cast<uint16_t*>(out),
                     ldo, vec_store, int32_t(n_big), int32_t(grid_big));
  return hipGetLastError();
}

}  // namespace nvfp4
