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
// Two ways to finish a last round that would leave CUs idle:
//  * halves (no workspace): when the last round would be at most half full,
//    its tiles are split into two 128-row halves each, which take about half
//    as long;
//  * stream-K (with a workspace): the 64-k steps of the remaining tiles are
//    dealt out evenly, as contiguous ranges in tile order, to one workgroup
//    per CU.  A tile cut between several workgroups is finished by the one
//    holding its last step: it adds the others' fp32 partial tiles, in a
//    fixed order, to its own.  Each workgroup walks its range last tile
//    first, so the partial it publishes (the head of its last tile) is ready
//    early, and it only ever waits on lower-numbered workgroups: workgroups
//    are dispatched in order, so the lowest unfinished one is always running
//    and never waits, and the launch cannot deadlock.
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
// kCpol != 0: global stores with that cache policy (output under 2 GiB).
template <int BMT, int kCpol = 0, typename Chunk>
__device__ __forceinline__ void w4a4_store(_Float16* __restrict__ lds, Chunk chunk, int32_t M, int32_t N,
                                           uint16_t* __restrict__ out, int64_t ldo, int vec_store, int32_t tb,
                                           int32_t m0) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  if (vec_store) {
    gemm::store_tile_lds<BMT, kCpol>(lds, chunk, out, ldo, m0, M, 16 * tb, N);
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
          const uint16_t bits = __builtin_bit_cast(uint16_t, (__bf16)vv[e]);
          if (kCpol != 0)
            __builtin_amdgcn_raw_buffer_store_b16(bits, gemm::buffer_rsrc(out), int32_t((int64_t(m) * ldo + n) * 2), 0,
                                                  kCpol);
          else
            orow[n] = bits;
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

// acc of one tile over the steps [sb, se).
template <int BMT>
__device__ __forceinline__ void w4a4_mma(gemm::AccT<BMT>& acc, _Float16* __restrict__ lds,
                                         const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, int32_t M,
                                         const uint8_t* __restrict__ wt, int32_t N, int32_t K, int32_t tb,
                                         int32_t m0, int32_t sb, int32_t se) {
  const int wn = int(threadIdx.x >> 6) & 1;
  const int32_t tiles = (N + 15) / 16;
  gemm::mainloop<false, BMT>(
      acc, lds, ac, as, [&](int i) { return int64_t(min(m0 + i, M - 1)); }, wt,
      [&](int lt) { return int64_t(min(tb + lt, tiles - 1)); }, [&](int t) { return 128 * wn + 32 * t; }, K, sb, se);
}

template <int BMT>
__device__ __forceinline__ void w4a4_tile(_Float16* __restrict__ lds, const uint8_t* __restrict__ ac,
                                          const uint8_t* __restrict__ as, int32_t M, const uint8_t* __restrict__ wt,
                                          int32_t N, int32_t K, float alpha, uint16_t* __restrict__ out, int64_t ldo,
                                          int vec_store, int32_t nblk, int32_t m0) {
  const int32_t tb = nblk * (gemm::BN / 16);  // first weight tile of the workgroup
  gemm::AccT<BMT> acc;
  w4a4_mma<BMT>(acc, lds, ac, as, M, wt, N, K, tb, m0, 0, -1);
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

// ------------------------------------------------------------------ stream-K
// Workspace: G partial tiles of 256 x 256 fp32 (in accumulator-register
// order: float4 c = 4*(2t + u) + i/4 of thread tid at c*512 + tid), then G
// int32 flags (1 = partial published; the consumer clears it, so the flags
// are all zero between launches), then one int32 count of timed-out waits.
constexpr int64_t kPartialBytes = int64_t(gemm::BN) * gemm::BM * 4;
// Leftover tiles are cut into about kMaxSplit pieces at most; the workgroup
// finishing a tile adds at most kMaxPartials partials (the host plan checks
// it for the ranges it picks).
constexpr int kMaxSplit = 4;
constexpr int kMaxPartials = 5;
constexpr int kSpinLimit = 1 << 22;  // bounded wait (s_sleep 4 each): about a second

__host__ __device__ inline int64_t sk_begin(int32_t j, int64_t units, int32_t G) { return int64_t(j) * units / G; }

// The workgroup whose range holds unit u.
__host__ __device__ inline int32_t sk_owner(int64_t u, int64_t units, int32_t G) {
  int32_t j = int32_t(u * G / units);
  while (j + 1 < G && sk_begin(j + 1, units, G) <= u) ++j;
  while (j > 0 && sk_begin(j, units, G) > u) --j;
  return j;
}

// Partials and flags are exchanged between workgroups on different XCDs,
// whose L2 caches are not coherent with each other.
//  * publish: every wave writes its part of the partial with system-scope
//    stores (sc0 sc1, written through) and takes an agent-scope release (an
//    L2 write-back queued behind its own stores), then one atomic swap
//    raises the flag;
//  * finish: the flags are taken with compare-and-swap (1 -> 0), then every
//    wave takes an agent-scope acquire (invalidating its L1 and its XCD's
//    L2) and reads the partials with ordinary loads.
// Every flag access is a read-modify-write atomic, which the device resolves
// coherently (a plain load could hit a stale line of a fresh workspace).  The
// finishing workgroups write their output through as well, so the
// write-backs (which stall the XCD's L2) find little to write.
constexpr int kSysScope = 1 | 16;  // sc0 | sc1

__device__ __forceinline__ void sk_store_partial(const gemm::Acc& acc, __amdgpu_buffer_rsrc_t rsrc, int32_t slot) {
  const int tid = int(threadIdx.x);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4_t v = {__float_as_uint(acc.v[t][u][4 * c]), __float_as_uint(acc.v[t][u][4 * c + 1]),
                           __float_as_uint(acc.v[t][u][4 * c + 2]), __float_as_uint(acc.v[t][u][4 * c + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, ((4 * (2 * t + u) + c) * gemm::kThreads + tid) * 16,
                                               slot * int32_t(kPartialBytes), kSysScope);
      }
}

// Steps [sb, se) of leftover tile r (tile n_full + r of the grouped order),
// run by remainder workgroup j: publishes a partial (se < steps) or finishes
// the tile (se == steps), adding the partials of the lower-numbered
// workgroups holding its steps [0, sb).
__device__ __forceinline__ void sk_segment(_Float16* __restrict__ lds, const uint8_t* __restrict__ ac,
                                        const uint8_t* __restrict__ as, int32_t M, const uint8_t* __restrict__ wt,
                                        int32_t N, int32_t K, float alpha, uint16_t* __restrict__ out, int64_t ldo,
                                        int vec_store, int32_t n_full, int32_t r, int32_t sb, int32_t se, int32_t j,
                                        int32_t jf, float4* __restrict__ partials, int32_t* __restrict__ flags,
                                        int32_t* __restrict__ timeouts) {
  const int32_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  const int32_t steps = K / gemm::BK;
  int32_t nblk, mblk;
  gemm::grouped_tile(n_full + r, nt, mt, nblk, mblk);
  const int32_t tb = nblk * (gemm::BN / 16), m0 = mblk * gemm::BM;
  gemm::Acc acc;
  w4a4_mma<gemm::BM>(acc, lds, ac, as, M, wt, N, K, tb, m0, sb, se);
  const __amdgpu_buffer_rsrc_t prsrc = gemm::buffer_rsrc(partials);
  if (se < steps) {
    sk_store_partial(acc, prsrc, j);
    // each wave's own release: its write-back is queued behind its stores
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_exchange(flags + j, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (sb > 0) {
      if (threadIdx.x == 0) {
        for (int32_t jp = j - 1; jp >= jf; --jp) {
          // take the flag (1 -> 0) in one compare-and-swap
          for (int n = 0;; ++n) {
            int32_t expected = 1;
            if (__hip_atomic_compare_exchange_strong(flags + jp, &expected, 0, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
              break;
            if (n >= kSpinLimit) {
              atomicAdd(timeouts, 1);
              break;
            }
            __builtin_amdgcn_s_sleep(4);
          }
        }
      }
      __syncthreads();  // every flag seen
      // each wave invalidates its L1 and its XCD's L2 before reading: a clean
      // but stale copy of a partial (say from the workspace's fill) could
      // still be cached there, and system-scope loads do not bypass it
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    // own sum plus the partials of workgroups j-1 down to jf (a fixed order),
    // added chunk by chunk as the tile is stored (the adds are unrolled over
    // at most kMaxPartials partials, so loads of several chunks overlap).
    // Only awaited partials are ever read: the unrolled loads past the np
    // real ones re-read partial j-1 and are discarded.
    const int tid = int(threadIdx.x);
    const int np = j - jf;
    if (np == 0) {
      w4a4_store<gemm::BM, kSysScope>(
          lds, [&](int t, int u, int g) { return acc_chunk<gemm::BM>(acc, t, u, g, alpha); }, M, N, out, ldo,
          vec_store, tb, m0);
    } else {
      w4a4_store<gemm::BM, kSysScope>(
          lds,
          [&](int t, int u, int g) {
            float4 v = make_float4(acc.v[t][u][4 * g], acc.v[t][u][4 * g + 1], acc.v[t][u][4 * g + 2],
                                   acc.v[t][u][4 * g + 3]);
            const int32_t voff = ((4 * (2 * t + u) + g) * gemm::kThreads + tid) * 16;
#pragma unroll
            for (int k = 0; k < kMaxPartials; ++k) {
              const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(
                  prsrc, voff, (j - 1 - min(k, np - 1)) * int32_t(kPartialBytes), 0);
              const bool take = k < np;
              v.x = take ? v.x + __uint_as_float(q[0]) : v.x;
              v.y = take ? v.y + __uint_as_float(q[1]) : v.y;
              v.z = take ? v.z + __uint_as_float(q[2]) : v.z;
              v.w = take ? v.w + __uint_as_float(q[3]) : v.w;
            }
            return make_float4(v.x * alpha, v.y * alpha, v.z * alpha, v.w * alpha);
          },
          M, N, out, ldo, vec_store, tb, m0);
    }
  }
  __syncthreads();  // a following segment reuses the LDS
}

// Workgroups [0, grid_full) run the first n_full tiles of the grouped order
// whole (XCD-aware); workgroup grid_full + j (j < G) runs the units
// [j*U/G, (j+1)*U/G) of the remaining tiles, U = their count x K/64 steps.
// G >= the number of remaining tiles, so a range spans at most two tiles:
// the head of the later one runs first.
__global__ __launch_bounds__(gemm::kThreads) void w4a4_sk_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, int32_t M, const uint8_t* __restrict__ wt,
    int32_t N, int32_t K, const float* __restrict__ alpha_p, uint16_t* __restrict__ out, int64_t ldo, int vec_store,
    int32_t n_full, int32_t grid_full, int32_t G, float4* __restrict__ partials, int32_t* __restrict__ flags,
    int32_t* __restrict__ timeouts) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  const int32_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  const float alpha = *alpha_p;
  const int32_t id = int32_t(blockIdx.x);
  if (id < grid_full) {
    int32_t nblk, mblk;
    if (!gemm::xcd_tile(id, nt, mt, n_full, nblk, mblk)) return;
    w4a4_tile<gemm::BM>(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, nblk, mblk * gemm::BM);
    return;
  }
  const int32_t j = id - grid_full;
  const int32_t steps = K / gemm::BK;
  const int64_t units = int64_t(nt * mt - n_full) * steps;
  if (j >= G) return;
  const int64_t u0 = sk_begin(j, units, G), u1 = sk_begin(j + 1, units, G);
  if (u0 >= u1) return;
  const int32_t r0 = int32_t(u0 / steps), r1 = int32_t((u1 - 1) / steps);
  if (r1 != r0)  // head of the later tile: a partial for the workgroup finishing it
    sk_segment(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, n_full, r1, 0, int32_t(u1 - int64_t(r1) * steps),
               j, j, partials, flags, timeouts);
  const int64_t t0 = int64_t(r0) * steps;
  const int32_t se = int32_t(min(u1, t0 + steps) - t0);
  sk_segment(lds, ac, as, M, wt, N, K, alpha, out, ldo, vec_store, n_full, r0, int32_t(u0 - t0), se, j,
             se == steps && u0 > t0 ? sk_owner(t0, units, G) : j, partials, flags, timeouts);
}

// Stream-K plan for the tiles left over by whole rounds: used when there are
// whole rounds and a leftover of at most 4/5 of a round, or when the whole
// problem is at most a quarter of a round (each tile is then cut into
// several pieces); not when the tiles fill a round part-way without a whole
// round before them (there the exchange of partials costs more than the
// balance gains).  At most kMaxSplit pieces per leftover tile.

struct SkPlan {
  int64_t n_full, G;
};

SkPlan sk_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t total = ((N + gemm::BN - 1) / gemm::BN) * ((M + gemm::BM - 1) / gemm::BM);
  const int64_t cus = device_cu_count();
  const int64_t rest = total % cus, steps = K / gemm::BK;
  const bool rounds = total > cus && 5 * rest <= 4 * cus, small = 4 * total <= cus;
  if (rest == 0 || !(rounds || small)) return SkPlan{total, 0};
  // G >= rest: no range spans more than two tiles
  int64_t G = std::min<int64_t>({cus, rest * kMaxSplit, rest * steps});
  const int64_t units = rest * steps;
  for (; G > rest; --G) {
    int64_t worst = 0;  // most partials any leftover tile needs
    for (int64_t r = 0; r < rest; ++r)
      worst = std::max<int64_t>(worst, sk_owner(r * steps + steps - 1, units, int32_t(G)) -
                                           sk_owner(r * steps, units, int32_t(G)));
    if (worst <= kMaxPartials) break;
  }
  return SkPlan{total - rest, G};
}

}  // namespace

int64_t w4a4_workspace_bytes() {
  const int64_t cus = device_cu_count();
  return cus * kPartialBytes + 4 * cus + 256;
}

// The stream-K finish is switched off: now and then a finishing workgroup
// summed a partial that was not the one just published (two calls on the
// same inputs gave different bits, each time right after another kernel had
// overwritten the partial slots).  Its flags protocol never timed out, so the
// read-modify-write atomics were coherent across XCDs, but the partial reads
// after the agent-scope acquire were not always.  Until the exchange no
// longer depends on that acquire, the workspace entry point runs the
// one-launch kernel (same bits as the call without a workspace).
constexpr bool kStreamKFinish = false;

hipError_t launch_w4a4_sk(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                          int64_t K, const float* alpha, void* out, int64_t ldo, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // (the stream-K stores use 32-bit byte offsets into out)
  const SkPlan plan =
      kStreamKFinish && M * ldo * 2 < (int64_t(1) << 31) ? sk_plan(M, N, K) : SkPlan{0, 0};
  if (plan.G == 0) return launch_w4a4(a_codes, a_scales, M, w_tiled, N, K, alpha, out, ldo, stream);
  const int64_t cus = device_cu_count();
  auto* partials = static_cast<float4*>(ws);
  auto* flags = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + cus * kPartialBytes);
  const int64_t grid_full = plan.n_full > 0 ? gemm::xcd_grid(int32_t(plan.n_full)) : 0;
  const int vec_store = (reinterpret_cast<uintptr_t>(out) % 16 == 0 && (ldo * 2) % 16 == 0) ? 1 : 0;
  hipLaunchKernelGGL(w4a4_sk_kernel, dim3(uint32_t(grid_full + plan.G)), dim3(gemm::kThreads), 0, stream,
                     static_cast<const uint8_t*>(a_codes), static_cast<const uint8_t*>(a_scales), int32_t(M),
                     static_cast<const uint8_t*>(w_tiled), int32_t(N), int32_t(K), alpha, static_cast<uint16_t*>(out),
                     ldo, vec_store, int32_t(plan.n_full), int32_t(grid_full), int32_t(plan.G), partials, flags,
                     flags + cus);
  return hipGetLastError();
}

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
