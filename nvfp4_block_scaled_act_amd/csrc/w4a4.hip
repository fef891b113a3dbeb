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
//
// A batch of at most 128 rows runs on its own kernel (w4a4_skinny_kernel): each
// wave dequantizes its weight rows straight into MFMA operand registers and
// only the activation tile goes through LDS, so the weight stream, not the
// LDS staging of a mostly empty 256 x 256 tile, sets the pace (N = 62080,
// K = 5120: 81 -> 37 us at M <= 32, 88 -> 54 us at M = 64).
//
// Few tiles (a small batch on a weight of a few thousand rows: N = 8704 has
// 34 column tiles, so 34 of 256 CUs would work through all of K) split K
// across workgroups when the caller provides room for fp32 partials: tile x
// range workgroups each run the main loop over their range of whole 256-k
// units and store an fp32 partial tile; a second launch adds the ranges'
// partials in range order (a fixed fp32 sum order), scales by alpha and
// rounds once to bf16.
#include "gemm_skinny.hpp"
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
// 256-row tiles (XCD-aware); the rest run the remaining tiles as two 128-row
// halves each.
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
    const int32_t m0 = mblk * gemm::BM + (gemm::BM / 2) * (j % 2);
    if (m0 >= M) return;
    w4a4_tile<gemm::BM / 2>(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, nblk, m0);
  }
}

// ---------------------------------------------------------------- split K
// fp32 partial of tile (nblk, m0) over the 256-k units [u0, u1): stored
// unscaled at part[m][n] (row-major [M, N]).  The operands run swapped in the
// MFMA, so register i of lane l in wave tile (t, u) holds weight row 16 tb +
// 128 wn + 32 t + l % 32 for activation row m0 + (BMT/4) wm + 32 u + 8 (i/4)
// + 4 (l/32) + i % 4, and each store instruction writes whole 128-byte rows
// pieces.
template <int BMT>
__device__ __forceinline__ void w4a4_partial_tile(_Float16* __restrict__ lds, const uint8_t* __restrict__ ac,
                                                  const uint8_t* __restrict__ as, int32_t M,
                                                  const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                  float* __restrict__ part, int32_t nblk, int32_t m0, int32_t u0,
                                                  int32_t u1) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1, h = lane >> 5;
  const int32_t tb = nblk * (gemm::BN / 16);
  const int32_t tiles = (N + 15) / 16;
  gemm::AccT<BMT> acc;
  gemm::mainloop<true, BMT>(
      acc, lds, ac, as, [&](int i) { return int64_t(min(m0 + i, M - 1)); }, wt,
      [&](int lt) { return int64_t(min(tb + lt, tiles - 1)); }, [&](int t) { return 128 * wn + 32 * t; }, K,
      2 * u0, 2 * (u1 - u0));
  const int32_t n = 16 * tb + 128 * wn + (lane & 31);
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t m = m0 + wm * (BMT / 4) + 32 * u + 8 * (i >> 2) + 4 * h + (i & 3);
      if (m >= M) continue;
      float* row = part + int64_t(m) * N;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (n + 32 * t < N) row[n + 32 * t] = acc.v[t][u][i];
    }
}

// Workgroup id -> (tile L = id % tiles of the grouped order, range s = id /
// tiles).
__global__ __launch_bounds__(gemm::kThreads) void w4a4_splitk_kernel(const uint8_t* __restrict__ ac,
                                                                     const uint8_t* __restrict__ as, int32_t M,
                                                                     const uint8_t* __restrict__ wt, int32_t N,
                                                                     int32_t K, float* __restrict__ partials,
                                                                     int32_t splits, int32_t tiles) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  const int32_t id = int32_t(blockIdx.x);
  const int32_t L = id % tiles, s = id / tiles;
  const int32_t units = K / 256;
  const int32_t u0 = int32_t(int64_t(s) * units / splits), u1 = int32_t(int64_t(s + 1) * units / splits);
  float* part = partials + int64_t(s) * M * N;
  const int32_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  int32_t nblk, mblk;
  gemm::grouped_tile(L, nt, mt, nblk, mblk);
  w4a4_partial_tile<gemm::BM>(lds, ac, as, M, wt, N, K, part, nblk, mblk * gemm::BM, u0, u1);
}

// out[m][n] = bf16(alpha * (part_0 + part_1 + ... + part_{splits-1})[m][n]),
// added in range order in fp32; four outputs of one row per thread.
__global__ __launch_bounds__(256) void w4a4_splitk_reduce_kernel(const float* __restrict__ partials, int32_t splits,
                                                                 int32_t M, int32_t N,
                                                                 const float* __restrict__ alpha_p,
                                                                 uint16_t* __restrict__ out, int64_t ldo) {
  const int32_t nq = (N + 3) / 4;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(M) * nq) return;
  const int32_t m = int32_t(i / nq), n = int32_t(i - int64_t(m) * nq) * 4;
  const float alpha = *alpha_p;
  const int64_t plane = int64_t(M) * N;
  const float* p = partials + int64_t(m) * N + n;
  uint16_t* o = out + int64_t(m) * ldo + n;
  if (N % 4 == 0) {  // whole 16-byte pieces (each row starts 16-byte aligned)
    float4 a = *reinterpret_cast<const float4*>(p);
    for (int32_t s = 1; s < splits; ++s) {
      const float4 b = *reinterpret_cast<const float4*>(p + s * plane);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const uint2 v = make_uint2(pack_bf16x2(a.x * alpha, a.y * alpha), pack_bf16x2(a.z * alpha, a.w * alpha));
    if ((reinterpret_cast<uintptr_t>(o) & 7) == 0) {
      *reinterpret_cast<uint2*>(o) = v;
    } else {
      o[0] = uint16_t(v.x);
      o[1] = uint16_t(v.x >> 16);
      o[2] = uint16_t(v.y);
      o[3] = uint16_t(v.y >> 16);
    }
    return;
  }
  for (int e = 0; e < 4 && n + e < N; ++e) {
    float a = p[e];
    for (int32_t s = 1; s < splits; ++s) a += p[s * plane + e];
    o[e] = __builtin_bit_cast(uint16_t, (__bf16)(a * alpha));
  }
}

// ---------------------------------------------------------------- few rows
// A batch of at most 128 rows: skinny::mainloop over 256 weight rows per
// workgroup (gemm_skinny.hpp).
// Workgroup id -> (row block blk = id % nblocks, K range s = id / nblocks).
// splits == 1: out[m][n] = bf16(alpha * acc); else the unscaled fp32 partial
// of range s at partials + s * M * N, row-major [M, N].
template <int G>
__global__ __launch_bounds__(skinny::kThreads) void w4a4_skinny_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, int32_t M, const uint8_t* __restrict__ wt,
    int32_t N, int32_t K, const float* __restrict__ alpha_p, uint16_t* __restrict__ out, int64_t ldo,
    float* __restrict__ partials, int32_t splits, int32_t nblocks) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[skinny::lds_halves<G>()];
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int32_t id = int32_t(blockIdx.x);
  const int32_t blk = id % nblocks, s = id / nblocks;
  const int32_t units = K / 256;
  const int32_t u0 = int32_t(int64_t(s) * units / splits), u1 = int32_t(int64_t(s + 1) * units / splits);
  const int32_t tiles16 = (N + 15) / 16, first16 = blk * (skinny::kRows / 16);
  f32x16_t acc[skinny::TW][G];
  skinny::mainloop<G, skinny::depth<G>()>(
      acc, lds, ac, as, [&](int i) { return int64_t(min(i, M - 1)); }, wt,
      [&](int j) { return int64_t(min(first16 + j, tiles16 - 1)); }, K, u0, u1);

  const int h = lane >> 5;
  const int32_t n = blk * skinny::kRows + 32 * skinny::TW * wave + (lane & 31);
  if (splits == 1) {
    const float alpha = *alpha_p;
#pragma unroll
    for (int t = 0; t < skinny::TW; ++t) {
      if (n + 32 * t >= N) continue;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t m = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
          if (m < M) out[int64_t(m) * ldo + n + 32 * t] = __builtin_bit_cast(uint16_t, (__bf16)(acc[t][g][i] * alpha));
        }
    }
  } else {
    float* part = partials + int64_t(s) * M * N;
#pragma unroll
    for (int t = 0; t < skinny::TW; ++t) {
      if (n + 32 * t >= N) continue;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t m = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
          if (m < M) part[int64_t(m) * N + n + 32 * t] = acc[t][g][i];
        }
    }
  }
}

}  // namespace

int w4a4_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 256) return 1;
  const int64_t units = K / 256;
  const int64_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  // one workgroup per 256-row column tile for a few rows (w4a4_skinny_kernel)
  const int64_t tiles = M <= skinny::kMaxM ? nt : nt * mt;
  const int64_t cus = device_cu_count();
  // only when the tiles fill at most half the CUs; at least two units per range
  if (units < 4 || 2 * tiles > cus) return 1;
  int64_t s = std::min<int64_t>({cus / tiles, units / 2, 16});
  // the partials stay within kSplitKMaxBytes and, with the dispatched
  // linear's quantized activations, within its allocation-free scratch
  const int64_t act = int64_t(linear_act_bytes(M, K));
  const int64_t budget = std::min<int64_t>(int64_t(kSplitKMaxBytes), int64_t(kLinearScratchBytes) - act - 256);
  const int64_t plane = M * N * 4;
  s = std::min<int64_t>(s, budget > 0 ? budget / plane : 0);
  return s >= 2 ? int(s) : 1;
}

size_t w4a4_partials_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = w4a4_splits(M, N, K);
  return s > 1 ? (size_t(s) * size_t(M) * size_t(N) * 4 + 255) / 256 * 256 : 0;
}

hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, float* partials, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* AC = static_cast<const uint8_t*>(a_codes);
  const auto* AS = static_cast<const uint8_t*>(a_scales);
  const auto* WT = static_cast<const uint8_t*>(w_tiled);
  auto* O = static_cast<uint16_t*>(out);
  const int64_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  const int splits = partials ? w4a4_splits(M, N, K) : 1;
  if (M <= skinny::kMaxM) {
    // few rows: 256 weight rows per workgroup (as many workgroups as 256-row
    // column tiles, so w4a4_splits applies unchanged)
    static_assert(skinny::kRows == gemm::BN, "one skinny workgroup per 256-row column tile");
    const dim3 grid(uint32_t(nt * splits)), block(skinny::kThreads);
    float* part = splits > 1 ? partials : nullptr;
    if (M <= 32)
      hipLaunchKernelGGL(w4a4_skinny_kernel<1>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
                         alpha, O, ldo, part, splits, int32_t(nt));
    else if (M <= 64)
      hipLaunchKernelGGL(w4a4_skinny_kernel<2>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
                         alpha, O, ldo, part, splits, int32_t(nt));
    else
      hipLaunchKernelGGL(w4a4_skinny_kernel<4>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
                         alpha, O, ldo, part, splits, int32_t(nt));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t threads = M * ((N + 3) / 4);
    hipLaunchKernelGGL(w4a4_splitk_reduce_kernel, dim3(uint32_t((threads + 255) / 256)), dim3(256), 0, stream,
                       partials, splits, int32_t(M), int32_t(N), alpha, O, ldo);
    return hipGetLastError();
  }
  if (splits > 1) {
    const int64_t tiles = nt * mt;
    hipLaunchKernelGGL(w4a4_splitk_kernel, dim3(uint32_t(tiles * splits)), dim3(gemm::kThreads), 0, stream, AC, AS,
                       int32_t(M), WT, int32_t(N), int32_t(K), partials, splits, int32_t(tiles));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = M * ((N + 3) / 4);
    hipLaunchKernelGGL(w4a4_splitk_reduce_kernel, dim3(uint32_t((threads + 255) / 256)), dim3(256), 0, stream,
                       partials, splits, int32_t(M), int32_t(N), alpha, O, ldo);
    return hipGetLastError();
  }
  const int64_t total = nt * mt;
  const int64_t cus = device_cu_count();
  const int64_t rest = total % cus;
  // split the last round into halves when it is at most half full
  const int64_t n_big = (total > cus && rest > 0 && 2 * rest <= cus) ? total - rest : total;
  const int64_t grid_big = n_big > 0 ? gemm::xcd_grid(int32_t(n_big)) : 0;
  const int64_t grid = grid_big + 2 * (total - n_big);
  // whole 16-byte output pieces when the rows are 16-byte aligned
  const int vec_store = (reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * 2) % 16 == 0) ? 1 : 0;
  hipLaunchKernelGGL(w4a4_kernel, dim3(uint32_t(grid)), dim3(gemm::kThreads), 0, stream, AC, AS, int32_t(M), WT,
                     int32_t(N), int32_t(K), alpha, O, ldo, vec_store, int32_t(n_big), int32_t(grid_big));
  return hipGetLastError();
}

}  // namespace nvfp4
