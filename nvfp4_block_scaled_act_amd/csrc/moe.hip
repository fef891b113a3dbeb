// NVFP4 MoE expert layer (W4A4 on both GEMMs) on gfx950.
//
// Layer flow (FreeToken PR #733, Changes: align, gate_up, activation, down,
// sum; FreeToken PR #736, Changes: both GEMMs take NVFP4 activations, the
// gate_up epilogue applies the gated activation and quantizes to NVFP4, the
// down epilogue applies the routing weight and sums the routes):
//   align    group the T*top_k (token, route) pairs by expert, stable in pair
//            order; cut each expert's segment into tiles of up to 256 pairs
//   gate_up  z = alpha_gu[e] * deq(q(x_t)) . deq(W_gu[e])^T   (2I outputs)
//            h = SiLU(z[:I]) * z[I:]  in fp32, quantized to NVFP4 with g2
//   down     y = alpha_dn[e] * deq(h) . deq(W_dn[e])^T       (K outputs)
//            ys[slot] = w[t, r] * y in fp32, by slot
//   sum      out[t] = bf16(sum_r ys[slot of (t, r)]), routes in order r = 0..
// (a fixed summation order: the layer's output bits are reproducible)
// Both GEMMs run gemm::mainloop on one 256-pair tile and 256 weight rows per
// workgroup.  The tile table has a fixed maximum length (every expert can
// leave one partial tile), so no launch depends on counts read back to the
// host; workgroups past the table's live entries exit at once.
#include <algorithm>

#include "gemm_skinny.hpp"
#include "gemm_w4a4.hpp"
#include "kernels.hpp"
#include "quant_exact.hpp"

namespace nvfp4 {

namespace {

constexpr int kChunk = 1024;  // pairs per align workgroup (one per thread)

// The pair's expert, or E for a pair that is skipped (id outside [0, E)).
__device__ __forceinline__ int expert_of(const int32_t* __restrict__ ids, int64_t p, int32_t E) {
  const int32_t e = ids[p];
  return (e >= 0 && e < E) ? e : E;
}

// counts[c][e] = pairs of chunk c routed to expert e.
// Also clears the h amax (when requested) for the gate_up kernel.
__global__ __launch_bounds__(kChunk) void moe_count_kernel(const int32_t* __restrict__ ids, int64_t P, int32_t E,
                                                           int32_t* __restrict__ counts, uint32_t* __restrict__ h_amax) {
  extern __shared__ int32_t cnt[];
  if (h_amax && blockIdx.x == 0 && threadIdx.x == 0) *h_amax = 0u;
  for (int e = int(threadIdx.x); e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int64_t p = int64_t(blockIdx.x) * kChunk + threadIdx.x;
  if (p < P) {
    const int e = expert_of(ids, p, E);
    if (e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = int(threadIdx.x); e < E; e += kChunk) counts[int64_t(blockIdx.x) * E + e] = cnt[e];
}

// Exclusive prefix sum over the 1024 threads of the workgroup (tmp: 16 ints).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* tmp, int32_t& total) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  total = 0;
  for (int w = 0; w < 16; ++w) {
    const int32_t t = tmp[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// One workgroup: per-expert totals, segment starts, the per-chunk bases the
// scatter adds its ranks to (written over the counts), and the tile table of
// up to tile_rows pairs per entry (256 for the W4A4 GEMMs, 16 for W4A16).
// When the [chunks, E] counts fit in kScanLdsInts, they are read into LDS
// with all threads at once and written back the same way, so each expert's
// thread walks its column in LDS instead of through dependent global loads.
constexpr int kScanLdsInts = 16384;

__global__ __launch_bounds__(1024) void moe_scan_kernel(int32_t* __restrict__ counts, int32_t chunks, int32_t E,
                                                        int32_t* __restrict__ offsets, MoeTile* __restrict__ tiles,
                                                        int32_t max_tiles, int32_t tile_rows) {
  extern __shared__ int32_t staged[];  // [chunks][E] if they fit, else unused
  __shared__ int32_t tmp[16];
  const int e = int(threadIdx.x);
  const int64_t n = int64_t(chunks) * E;
  const bool in_lds = n <= kScanLdsInts;  // the same test sizes the launch's LDS
  int32_t* col = in_lds ? staged : counts;
  if (in_lds) {
    for (int32_t i = e; i < int32_t(n); i += 1024) staged[i] = counts[i];
    __syncthreads();
  }
  int32_t total = 0;
  if (e < E) {
#pragma unroll 8
    for (int32_t c = 0; c < chunks; ++c) total += col[int64_t(c) * E + e];
  }
  const int32_t ntile = (total + tile_rows - 1) / tile_rows;
  int32_t pairs = 0, ntiles = 0;
  const int32_t seg = block_exclusive_scan(total, tmp, pairs);
  const int32_t tile0 = block_exclusive_scan(ntile, tmp, ntiles);
  if (e < E) {
    int32_t base = seg;
    for (int32_t c = 0; c < chunks; ++c) {
      const int64_t i = int64_t(c) * E + e;
      const int32_t v = col[i];
      col[i] = base;
      base += v;
    }
    offsets[e] = seg;
    for (int32_t j = 0; j < ntile; ++j) {
      MoeTile t;
      t.expert = e;
      t.slot0 = seg + tile_rows * j;
      t.rows = min(tile_rows, total - tile_rows * j);
      t.pad = 0;
      tiles[tile0 + j] = t;
    }
  }
  if (e == 0) offsets[E] = pairs;
  for (int32_t j = ntiles + e; j < max_tiles; j += 1024) tiles[j] = MoeTile{0, 0, 0, 0};
  if (in_lds) {
    __syncthreads();
    for (int32_t i = e; i < int32_t(n); i += 1024) counts[i] = staged[i];
  }
}

size_t scan_lds_bytes(int64_t chunks, int64_t E) {
  return chunks * E <= kScanLdsInts ? size_t(chunks * E) * sizeof(int32_t) : 0;
}

// sorted[base[c][e] + rank] = p, rank = number of earlier pairs of the chunk
// with the same expert (so the order within an expert is the pair order).
// inv[p] = the slot of pair p, -1 for a skipped pair.
__global__ __launch_bounds__(kChunk) void moe_scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int32_t E,
                                                             const int32_t* __restrict__ bases,
                                                             int32_t* __restrict__ sorted, int32_t* __restrict__ inv) {
  extern __shared__ int32_t wave_count[];  // [16][E]
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  for (int i = int(threadIdx.x); i < 16 * E; i += kChunk) wave_count[i] = 0;
  __syncthreads();
  const int64_t p = int64_t(blockIdx.x) * kChunk + threadIdx.x;
  const int e = p < P ? expert_of(ids, p, E) : E;
  // lanes of the wave with the same expert value: one ballot per bit
  uint64_t same = ~0ull;
  for (int b = 0; (1 << b) <= E; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ball = __ballot(bit);
    same &= bit ? ball : ~ball;
  }
  const uint64_t lower = same & ((1ull << lane) - 1ull);
  if (e < E && lower == 0) wave_count[wave * E + e] = __popcll(same);
  __syncthreads();
  if (e < E) {
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_count[w * E + e];
    const int32_t slot = bases[int64_t(blockIdx.x) * E + e] + before + __popcll(lower);
    sorted[slot] = int32_t(p);
    inv[p] = slot;
  } else if (p < P) {
    inv[p] = -1;
  }
}

__global__ void set_u32_kernel_moe(uint32_t* p) { *p = 0u; }

// The three align steps in one workgroup, for at most kChunk pairs (decode
// batches): the same results as count + scan + scatter (stable by pair within
// an expert), tile table entries of up to tile_rows pairs.
__global__ __launch_bounds__(kChunk) void moe_align_small_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                                 int32_t E, int32_t* __restrict__ offsets,
                                                                 MoeTile* __restrict__ tiles, int32_t max_tiles,
                                                                 int32_t tile_rows, int32_t* __restrict__ sorted,
                                                                 int32_t* __restrict__ inv) {
  extern __shared__ int32_t lds[];  // wave_count [16][E], then base [E]
  __shared__ int32_t tmp[16];
  int32_t* wave_count = lds;
  int32_t* base = lds + 16 * E;
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  for (int i = int(threadIdx.x); i < 16 * E; i += kChunk) wave_count[i] = 0;
  __syncthreads();
  const int64_t p = threadIdx.x;
  const int e = p < P ? expert_of(ids, p, E) : E;
  uint64_t same = ~0ull;
  for (int b = 0; (1 << b) <= E; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ball = __ballot(bit);
    same &= bit ? ball : ~ball;
  }
  const uint64_t lower = same & ((1ull << lane) - 1ull);
  if (e < E && lower == 0) wave_count[wave * E + e] = __popcll(same);
  __syncthreads();
  // per-expert totals, segment starts and tiles (thread = expert)
  const int ex = int(threadIdx.x);
  int32_t total = 0;
  if (ex < E)
    for (int w = 0; w < 16; ++w) total += wave_count[w * E + ex];
  const int32_t ntile = (total + tile_rows - 1) / tile_rows;
  int32_t pairs = 0, ntiles = 0;
  const int32_t seg = block_exclusive_scan(total, tmp, pairs);
  const int32_t tile0 = block_exclusive_scan(ntile, tmp, ntiles);
  if (ex < E) {
    base[ex] = seg;
    offsets[ex] = seg;
    for (int32_t j = 0; j < ntile; ++j) {
      MoeTile t;
      t.expert = ex;
      t.slot0 = seg + tile_rows * j;
      t.rows = min(tile_rows, total - tile_rows * j);
      t.pad = 0;
      tiles[tile0 + j] = t;
    }
  }
  if (ex == 0) offsets[E] = pairs;
  for (int32_t j = ntiles + ex; j < max_tiles; j += kChunk) tiles[j] = MoeTile{0, 0, 0, 0};
  __syncthreads();
  if (e < E) {
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_count[w * E + e];
    const int32_t slot = base[e] + before + __popcll(lower);
    sorted[slot] = int32_t(p);
    inv[p] = slot;
  } else if (p < P) {
    inv[p] = -1;
  }
}

// gate_up of one tile of pairs x 128 gate rows (block c, + the matching 128
// up rows) of its expert, with the SiLU gate and NVFP4 quantization of h.
// BMT = pair rows the workgroup computes (256, or 128 for a tile that fits);
// row_of(i) = the activation row of the tile's row i (h is stored by slot).
template <int BMT, class RowOf>
__device__ __forceinline__ void gate_up_tile(_Float16* __restrict__ lds, const MoeTile& tile, int32_t c,
                                             const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                             int32_t K, RowOf row_of, const uint8_t* __restrict__ wt, int32_t I,
                                             float alpha, float g2, uint8_t* __restrict__ hc,
                                             uint8_t* __restrict__ hs, uint32_t* __restrict__ h_amax) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1, h = lane >> 5;
  // LDS weight tiles 0..7: gate rows 128c..128c+127, 8..15: the up rows I + the same
  const int32_t gate_tile0 = tile.expert * (2 * I / 16) + 8 * c, up_tile0 = gate_tile0 + I / 16;
  gemm::AccT<BMT> acc;
  gemm::mainloop<false, BMT>(
      acc, lds, xc, xs, row_of, wt,
      [&](int lt) { return int64_t(lt < 8 ? gate_tile0 + lt : up_tile0 + lt - 8); },
      // the wave's tiles 0, 1 are gate rows 64wn..64wn+63, tiles 2, 3 the up rows under them
      [&](int t) { return t < 2 ? 64 * wn + 32 * t : 128 + 64 * wn + 32 * (t - 2); }, K);

  float hmax = 0.0f;
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u) {
    const int32_t m = wm * (BMT / 4) + 32 * u + (lane & 31);  // pair row of the tile
    const int64_t slot = int64_t(tile.slot0) + m;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // h of gate rows 8(i/4) + 4h + i%4 of the wave's 32-row tile t
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = silu(alpha * acc.v[t][u][i]) * (alpha * acc.v[t + 2][u][i]);
      // lane half h gathers the 16-row block h of the tile: it keeps its own
      // registers of that block and takes the partner half's
      float x[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float own = h ? v[8 + j] : v[j];
        const float recv = __shfl_xor(h ? v[j] : v[8 + j], 32, 64);
        const float lo = h ? recv : own, hi = h ? own : recv;
        x[(j & 4) * 2 + (j & 3)] = lo;
        x[(j & 4) * 2 + 4 + (j & 3)] = hi;
      }
      if (m < tile.rows) {
        uint32_t c0, c1;
        const uint32_t s = quantize16_fast(x, g2, c0, c1);
        const int32_t i0 = 128 * c + 64 * wn + 32 * t + 16 * h;  // first h element of the block
        *reinterpret_cast<uint2*>(hc + slot * (I / 2) + i0 / 2) = make_uint2(c0, c1);
        hs[slot * (I / 16) + i0 / 16] = uint8_t(s);
#pragma unroll
        for (int i = 0; i < 16; ++i) hmax = __builtin_fmaxf(hmax, __builtin_fabsf(x[i]));
      }
    }
  }
  if (h_amax) {
    uint32_t bits = __float_as_uint(hmax);
    for (int o = 32; o > 0; o >>= 1) bits = max(bits, uint32_t(__shfl_xor(int(bits), o, 64)));
    if (lane == 0) atomicMax(h_amax, bits);
  }
}

// The same gate_up for a tile of at most 32 G pairs, on skinny::mainloop:
// waves 0..3 compute the 128 gate rows, waves 4..7 the up rows under them;
// z goes through LDS (fp32, [gate | up][pair row][128 + 4]) so that each
// thread then gates and quantizes whole 16-element blocks of h.
template <int G, class RowOf>
__device__ __forceinline__ void gate_up_tile_few(_Float16* __restrict__ lds, const MoeTile& tile, int32_t c,
                                                 const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                 int32_t K, RowOf row_of, const uint8_t* __restrict__ wt, int32_t I,
                                                 float alpha, float g2, uint8_t* __restrict__ hc,
                                                 uint8_t* __restrict__ hs, uint32_t* __restrict__ h_amax) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6), h = lane >> 5;
  const int32_t gate_tile0 = tile.expert * (2 * I / 16) + 8 * c, up_tile0 = gate_tile0 + I / 16;
  f32x16_t acc[skinny::TW][G];
  skinny::mainloop<G, skinny::depth<G>()>(
      acc, lds, xc, xs, row_of, wt, [&](int j) { return int64_t(j < 8 ? gate_tile0 + j : up_tile0 + j - 8); }, K, 0,
      K / 256);
  // register i of lane l: pair row 32g + 8(i/4) + 4(l/32) + i%4, weight row
  // 32 wave + l%32 of the workgroup's 256 (the mainloop's final barrier frees
  // the LDS)
  constexpr int ZP = 128 + 4;
  float* z = reinterpret_cast<float*>(lds);
  const int col = 32 * (wave & 3) + (lane & 31);
  float* zw = z + (wave >> 2) * (32 * G * ZP) + col;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) zw[(32 * g + 8 * (i >> 2) + 4 * h + (i & 3)) * ZP] = acc[0][g][i];
  __syncthreads();
  float hmax = 0.0f;
  for (int task = int(threadIdx.x); task < 32 * G * 8; task += skinny::kThreads) {
    const int m = task >> 3, b = task & 7;  // pair row, 16-element block of the 128
    if (m >= tile.rows) continue;
    const float4* zg = reinterpret_cast<const float4*>(z + m * ZP + 16 * b);
    const float4* zu = reinterpret_cast<const float4*>(z + (32 * G + m) * ZP + 16 * b);
    float x[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 gv = zg[q], uv = zu[q];
      x[4 * q] = silu(alpha * gv.x) * (alpha * uv.x);
      x[4 * q + 1] = silu(alpha * gv.y) * (alpha * uv.y);
      x[4 * q + 2] = silu(alpha * gv.z) * (alpha * uv.z);
      x[4 * q + 3] = silu(alpha * gv.w) * (alpha * uv.w);
    }
    uint32_t c0, c1;
    const uint32_t sc = quantize16_fast(x, g2, c0, c1);
    const int64_t slot = int64_t(tile.slot0) + m;
    const int32_t i0 = 128 * c + 16 * b;  // first h element of the block
    *reinterpret_cast<uint2*>(hc + slot * (I / 2) + i0 / 2) = make_uint2(c0, c1);
    hs[slot * (I / 16) + i0 / 16] = uint8_t(sc);
#pragma unroll
    for (int i = 0; i < 16; ++i) hmax = __builtin_fmaxf(hmax, __builtin_fabsf(x[i]));
  }
  if (h_amax) {
    uint32_t bits = __float_as_uint(hmax);
    for (int o = 32; o > 0; o >>= 1) bits = max(bits, uint32_t(__shfl_xor(int(bits), o, 64)));
    if (lane == 0) atomicMax(h_amax, bits);
  }
}

// gate_up of any tile: the few-rows loop up to 128 pairs, else the 256 x 256
// main loop.
template <class RowOf>
__device__ __forceinline__ void gate_up_any(_Float16* __restrict__ lds, const MoeTile& tile, int32_t c,
                                            const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, int32_t K,
                                            RowOf row_of, const uint8_t* __restrict__ wt, int32_t I, float alpha,
                                            float g2, uint8_t* __restrict__ hc, uint8_t* __restrict__ hs,
                                            uint32_t* __restrict__ h_amax) {
  if (tile.rows <= 32)
    gate_up_tile_few<1>(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
  else if (tile.rows <= 64)
    gate_up_tile_few<2>(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
  else if (tile.rows <= 128)
    gate_up_tile_few<4>(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
  else
    gate_up_tile<gemm::BM>(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
}

// Workgroup -> (tile, 128-row block c of the expert's I gate rows) by
// gemm::xcd_row_block; tiles of at most 128 pairs take the few-rows loop.
__global__ __launch_bounds__(gemm::kThreads) void moe_gate_up_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, int32_t K, int32_t top_k,
    const int32_t* __restrict__ sorted, const MoeTile* __restrict__ tiles, int32_t max_tiles,
    const uint8_t* __restrict__ wt, int32_t I, const float* __restrict__ alpha_gu, const float* __restrict__ g2_p,
    uint8_t* __restrict__ hc, uint8_t* __restrict__ hs, uint32_t* __restrict__ h_amax) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  int32_t ty, c;
  gemm::xcd_row_block(int32_t(blockIdx.x), I / 128, ty, c);
  if (ty >= max_tiles) return;
  const MoeTile tile = tiles[ty];
  if (tile.rows == 0) return;
  const float alpha = alpha_gu[tile.expert], g2 = *g2_p;
  auto row_of = [&](int i) { return int64_t(sorted[tile.slot0 + min(i, tile.rows - 1)] / top_k); };
  gate_up_any(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
}

// The same gate_up on a dense batch (a gated MLP's first GEMM): row tile ty
// holds rows 256ty.. of the NVFP4 activations, h is stored by row.
// Workgroups [0, n_big) take (row tile, block) items by gemm::xcd_row_block;
// when the items leave a last round at most half full, its items run as two
// 128-row halves each: workgroup n_big + j takes half j % 2 of item
// n_big + j / 2.
__global__ __launch_bounds__(gemm::kThreads) void gated_mlp_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, int32_t K, int32_t M,
    const uint8_t* __restrict__ wt, int32_t I, const float* __restrict__ alpha_p, const float* __restrict__ g2_p,
    uint8_t* __restrict__ hc, uint8_t* __restrict__ hs, uint32_t* __restrict__ h_amax, int32_t n_big) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  const int32_t id = int32_t(blockIdx.x);
  const bool half = id >= n_big;
  int32_t ty, c;
  gemm::xcd_row_block(half ? n_big + (id - n_big) / 2 : id, I / 128, ty, c);
  if (ty >= (M + gemm::BM - 1) / gemm::BM) return;
  const int32_t m0 = ty * gemm::BM + (half ? (gemm::BM / 2) * ((id - n_big) & 1) : 0);
  if (m0 >= M) return;
  const MoeTile tile{0, m0, min(half ? gemm::BM / 2 : gemm::BM, M - m0), 0};
  const float alpha = *alpha_p, g2 = *g2_p;
  auto row_of = [&](int i) { return int64_t(tile.slot0 + min(i, tile.rows - 1)); };
  gate_up_any(lds, tile, c, xc, xs, K, row_of, wt, I, alpha, g2, hc, hs, h_amax);
}

// down of one tile of pairs x 256 outputs (block nblk of K) of its expert,
// scaled by alpha_dn[e] * w[pair] and stored by slot (fp32).
template <int BMT>
__device__ __forceinline__ void down_tile(_Float16* __restrict__ lds, const MoeTile& tile, int32_t nblk,
                                          const uint8_t* __restrict__ hc, const uint8_t* __restrict__ hs, int32_t I,
                                          const int32_t* __restrict__ sorted, const float* __restrict__ topk_w,
                                          int32_t top_k, const uint8_t* __restrict__ wt, int32_t K, float alpha,
                                          float* __restrict__ ys) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1, h = lane >> 5;
  const int32_t wtile0 = tile.expert * (K / 16) + nblk * 16;
  // the tile row's pair index, loaded before the main loop so that only the
  // routing weight's load is left for the epilogue (two dependent loads there
  // cost about 5 us per layer at T = 8192)
  int32_t pr = 0;
  if (threadIdx.x < BMT) pr = sorted[tile.slot0 + min(int(threadIdx.x), tile.rows - 1)];
  gemm::AccT<BMT> acc;
  gemm::mainloop<true, BMT>(
      acc, lds, hc, hs, [&](int i) { return int64_t(tile.slot0 + min(i, tile.rows - 1)); }, wt,
      [&](int lt) { return int64_t(wtile0 + lt); }, [&](int t) { return 128 * wn + 32 * t; }, I);

  // the tile's routing-weight scales, through LDS (free after the main loop)
  float* s_scale = reinterpret_cast<float*>(lds);
  if (threadIdx.x < BMT) s_scale[threadIdx.x] = alpha * topk_w[pr];
  __syncthreads();
  const int32_t n = nblk * 256 + 128 * wn + (lane & 31);
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = wm * (BMT / 4) + 32 * u + 8 * (i >> 2) + 4 * h + (i & 3);
      if (m >= tile.rows) continue;
      float* row = ys + (int64_t(tile.slot0) + m) * K + n;
      const float sc = s_scale[m];
#pragma unroll
      for (int t = 0; t < 4; ++t) row[32 * t] = sc * acc.v[t][u][i];
    }
}

// The same down for a tile of at most 32 G pairs, on skinny::mainloop:
// register i of lane l holds pair row 32g + 8(i/4) + 4(l/32) + i%4 and output
// 256 nblk + 32 wave + l%32, so each store writes 32 consecutive outputs.
template <int G>
__device__ __forceinline__ void down_tile_few(_Float16* __restrict__ lds, const MoeTile& tile, int32_t nblk,
                                              const uint8_t* __restrict__ hc, const uint8_t* __restrict__ hs,
                                              int32_t I, const int32_t* __restrict__ sorted,
                                              const float* __restrict__ topk_w, const uint8_t* __restrict__ wt,
                                              int32_t K, float alpha, float* __restrict__ ys) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6), h = lane >> 5;
  const int32_t wtile0 = tile.expert * (K / 16) + nblk * 16;
  int32_t pr = 0;  // the row's pair, loaded before the main loop
  if (threadIdx.x < 32 * G) pr = sorted[tile.slot0 + min(int(threadIdx.x), tile.rows - 1)];
  f32x16_t acc[skinny::TW][G];
  skinny::mainloop<G, skinny::depth<G>()>(
      acc, lds, hc, hs, [&](int i) { return int64_t(tile.slot0 + min(i, tile.rows - 1)); }, wt,
      [&](int j) { return int64_t(wtile0 + j); }, I, 0, I / 256);
  float* s_scale = reinterpret_cast<float*>(lds);
  if (threadIdx.x < 32 * G) s_scale[threadIdx.x] = alpha * topk_w[pr];
  __syncthreads();
  const int32_t n = nblk * 256 + 32 * wave + (lane & 31);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
      if (m < tile.rows) ys[(int64_t(tile.slot0) + m) * K + n] = s_scale[m] * acc[0][g][i];
    }
}

// Workgroup -> (tile, 256-output block of K) by gemm::xcd_row_block; tiles of
// at most 128 pairs take the few-rows loop.
__global__ __launch_bounds__(gemm::kThreads) void moe_down_kernel(
    const uint8_t* __restrict__ hc, const uint8_t* __restrict__ hs, int32_t I, const int32_t* __restrict__ sorted,
    const MoeTile* __restrict__ tiles, int32_t max_tiles, const float* __restrict__ topk_w, int32_t top_k,
    const uint8_t* __restrict__ wt, int32_t K, const float* __restrict__ alpha_dn, float* __restrict__ ys) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[gemm::kLdsHalves];
  int32_t ty, nblk;
  gemm::xcd_row_block(int32_t(blockIdx.x), K / 256, ty, nblk);
  if (ty >= max_tiles) return;
  const MoeTile tile = tiles[ty];
  if (tile.rows == 0) return;
  const float alpha = alpha_dn[tile.expert];
  if (tile.rows <= 32)
    down_tile_few<1>(lds, tile, nblk, hc, hs, I, sorted, topk_w, wt, K, alpha, ys);
  else if (tile.rows <= 64)
    down_tile_few<2>(lds, tile, nblk, hc, hs, I, sorted, topk_w, wt, K, alpha, ys);
  else if (tile.rows <= 128)
    down_tile_few<4>(lds, tile, nblk, hc, hs, I, sorted, topk_w, wt, K, alpha, ys);
  else
    down_tile<gemm::BM>(lds, tile, nblk, hc, hs, I, sorted, topk_w, top_k, wt, K, alpha, ys);
}

// out[t][k] = bf16(sum over the token's routes r = 0.. of ys[inv[t*top_k + r]][k])
// in fp32, four outputs per thread; skipped routes (inv < 0) add nothing.
// TK > 0: top_k == TK, and the loads of all the token's routes are issued
// before the sum (a skipped route re-reads slot 0 and is not added); TK == 0:
// any top_k, one route at a time.  Same sum order either way.  ys is read
// once, with nontemporal loads (measured on the T = 8192, top-8, K = 2048
// layer: 126 -> 92 us for its 539 MB, the streaming-read rate).
__device__ __forceinline__ float4 ld16f_nt(const float* p) {
  const uint4 v = ld16_nt(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

template <int TK>
__global__ __launch_bounds__(256) void moe_sum_kernel(const float* __restrict__ ys, const int32_t* __restrict__ inv,
                                                      int64_t T, int32_t top_k, int32_t K, uint16_t* __restrict__ out,
                                                      int64_t ldo) {
  const int64_t per_row = K / 4;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= T * per_row) return;
  const int64_t t = i / per_row, k = (i - t * per_row) * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (TK > 0) {
    int32_t slot[TK > 0 ? TK : 1];
    float4 x[TK > 0 ? TK : 1];
#pragma unroll
    for (int r = 0; r < TK; ++r) slot[r] = inv[t * TK + r];
#pragma unroll
    for (int r = 0; r < TK; ++r) x[r] = ld16f_nt(ys + int64_t(max(slot[r], 0)) * K + k);
#pragma unroll
    for (int r = 0; r < TK; ++r) {
      const bool take = slot[r] >= 0;
      a.x = take ? a.x + x[r].x : a.x;
      a.y = take ? a.y + x[r].y : a.y;
      a.z = take ? a.z + x[r].z : a.z;
      a.w = take ? a.w + x[r].w : a.w;
    }
  } else {
    for (int32_t r = 0; r < top_k; ++r) {
      const int32_t slot = inv[t * top_k + r];
      if (slot < 0) continue;
      const float4 x = ld16f_nt(ys + int64_t(slot) * K + k);
      a.x += x.x;
      a.y += x.y;
      a.z += x.z;
      a.w += x.w;
    }
  }
  *reinterpret_cast<uint2*>(out + t * ldo + k) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
}

// out[t] = bf16(sum of the token's routes in the order r = 0, 1, ...).
hipError_t launch_route_sum(const float* ys, const int32_t* inv, int64_t T, int64_t top_k, int64_t K, void* out,
                            int64_t ldo, hipStream_t stream) {
  const dim3 sum_grid{uint32_t((T * (K / 4) + 255) / 256)};
#define NVFP4_SUM(TK)                                                                                            \
  hipLaunchKernelGGL(moe_sum_kernel<TK>, sum_grid, dim3(256), 0, stream, ys, inv, T, int32_t(top_k), int32_t(K), \
                     static_cast<uint16_t*>(out), ldo)
  switch (top_k) {
    case 1: NVFP4_SUM(1); break;
    case 2: NVFP4_SUM(2); break;
    case 4: NVFP4_SUM(4); break;
    case 6: NVFP4_SUM(6); break;
    case 8: NVFP4_SUM(8); break;
    default: NVFP4_SUM(0); break;
  }
#undef NVFP4_SUM
  return hipGetLastError();
}

}  // namespace

MoeLayout moe_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  MoeLayout L{};
  const int64_t P = T * top_k;
  L.chunks = (P + kChunk - 1) / kChunk;
  L.max_tiles = P / gemm::BM + E;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  L.x_codes = take(T * K / 2);
  L.x_scales = take(T * K / 16);
  L.counts = take(4 * L.chunks * E);
  L.offsets = take(4 * (E + 1));
  L.tiles = take(int64_t(sizeof(MoeTile)) * L.max_tiles);
  L.sorted = take(4 * P);
  L.h_codes = take(P * I / 2);
  L.h_scales = take(P * I / 16);
  L.inv = take(4 * P);
  L.ys = take(4 * P * K);
  L.total = off;
  return L;
}

hipError_t launch_moe_w4a4(const void* x, int64_t T, int64_t ldx, const int32_t* ids, const float* topk_w,
                           int64_t top_k, int64_t E, int64_t I, const void* w_gate_up, const void* w_down, int64_t K,
                           const float* g1, const float* g2, const float* alpha_gu, const float* alpha_dn, void* out,
                           int64_t ldo, void* ws, float* h_amax, hipStream_t stream) {
  const MoeLayout L = moe_layout(T, top_k, E, K, I);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* xc = base + L.x_codes;
  uint8_t* xs = base + L.x_scales;
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  MoeTile* tiles = reinterpret_cast<MoeTile*>(base + L.tiles);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  uint8_t* hc = base + L.h_codes;
  uint8_t* hs = base + L.h_scales;
  int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
  float* ys = reinterpret_cast<float*>(base + L.ys);
  const int64_t P = T * top_k;
  hipError_t err = launch_quantize(x, T, K, ldx, g1, xc, xs, stream);
  if (err != hipSuccess) return err;
  const uint32_t chunks = uint32_t(L.chunks);
  hipLaunchKernelGGL(moe_count_kernel, dim3(chunks), dim3(kChunk), size_t(4 * E), stream, ids, P, int32_t(E), counts,
                     reinterpret_cast<uint32_t*>(h_amax));
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), scan_lds_bytes(L.chunks, E), stream, counts,
                     int32_t(L.chunks), int32_t(E), offsets, tiles, int32_t(L.max_tiles), int32_t(gemm::BM));
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(chunks), dim3(kChunk), size_t(4 * 16 * E), stream, ids, P, int32_t(E),
                     counts, sorted, inv);
  const int32_t mt = int32_t(L.max_tiles);
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(uint32_t(gemm::xcd_rows_grid(mt, int32_t(I / 128)))),
                     dim3(gemm::kThreads), 0, stream, xc, xs, int32_t(K), int32_t(top_k), sorted, tiles, mt,
                     static_cast<const uint8_t*>(w_gate_up), int32_t(I), alpha_gu, g2, hc, hs,
                     reinterpret_cast<uint32_t*>(h_amax));
  hipLaunchKernelGGL(moe_down_kernel, dim3(uint32_t(gemm::xcd_rows_grid(mt, int32_t(K / 256)))),
                     dim3(gemm::kThreads), 0, stream, hc, hs, int32_t(I), sorted, tiles, mt, topk_w, int32_t(top_k),
                     static_cast<const uint8_t*>(w_down), int32_t(K), alpha_dn, ys);
  return launch_route_sum(ys, inv, T, top_k, K, out, ldo, stream);
}

MoeW4A16Layout moe_w4a16_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  MoeW4A16Layout L{};
  const int64_t P = T * top_k;
  L.chunks = (P + kChunk - 1) / kChunk;
  L.max_tiles = P / kW4A16Rows + E;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  L.counts = take(4 * L.chunks * E);
  L.offsets = take(4 * (E + 1));
  L.tiles = take(int64_t(sizeof(MoeTile)) * L.max_tiles);
  L.sorted = take(4 * P);
  L.h = take(2 * P * I);
  L.inv = take(4 * P);
  L.ys = take(4 * P * K);
  L.total = off;
  return L;
}

hipError_t launch_moe_w4a16(const void* x, int64_t T, int64_t ldx, const int32_t* ids, const float* topk_w,
                            int64_t top_k, int64_t E, int64_t I, const void* w_gate_up, const void* w_down,
                            int64_t K, const float* alpha_gu, const float* alpha_dn, void* out, int64_t ldo, void* ws,
                            hipStream_t stream) {
  const MoeW4A16Layout L = moe_w4a16_layout(T, top_k, E, K, I);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  MoeTile* tiles = reinterpret_cast<MoeTile*>(base + L.tiles);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + L.h);
  int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
  float* ys = reinterpret_cast<float*>(base + L.ys);
  const int64_t P = T * top_k;
  if (P <= kMoeDirectPairs && top_k <= 16 && I / 256 <= 8) {
    // few pairs: each its own entry, no align, down and the route sum in one
    // launch (measured cold at E = 128, top-8, K = 2048, I = 768: T = 1/2/4/8
    // 15.9/19.1/24.9/34.3 -> 10.6/13.1/18.8/30.5 us; at T = 16, 128 pairs, the
    // grouped path is faster: 47.5 against 52.9 us)
    return launch_w4a16_moe_direct(x, ldx, ids, T, top_k, E, I, w_gate_up, w_down, K, alpha_gu, alpha_dn, topk_w,
                                   h, out, ldo, stream);
  }
  const uint32_t chunks = uint32_t(L.chunks);
  if (P <= kChunk && 17 * 4 * E <= 65536) {
    hipLaunchKernelGGL(moe_align_small_kernel, dim3(1), dim3(kChunk), size_t(4 * 17 * E), stream, ids, P, int32_t(E),
                       offsets, tiles, int32_t(L.max_tiles), int32_t(kW4A16Rows), sorted, inv);
  } else {
    hipLaunchKernelGGL(moe_count_kernel, dim3(chunks), dim3(kChunk), size_t(4 * E), stream, ids, P, int32_t(E), counts,
                       nullptr);
    hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), scan_lds_bytes(L.chunks, E), stream, counts,
                       int32_t(L.chunks), int32_t(E), offsets, tiles, int32_t(L.max_tiles), int32_t(kW4A16Rows));
    hipLaunchKernelGGL(moe_scatter_kernel, dim3(chunks), dim3(kChunk), size_t(4 * 16 * E), stream, ids, P,
                       int32_t(E), counts, sorted, inv);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // every live entry holds at least one pair
  const int64_t entries = std::min<int64_t>(L.max_tiles, P);
  err = launch_w4a16_grouped(true, x, ldx, sorted, top_k, tiles, entries, I / 16, w_gate_up, 2 * I, K, alpha_gu,
                             nullptr, h, I, stream);
  if (err != hipSuccess) return err;
  err = launch_w4a16_grouped(false, h, I, sorted, top_k, tiles, entries, K / 16, w_down, K, I, alpha_dn, topk_w, ys,
                             K, stream);
  if (err != hipSuccess) return err;
  return launch_route_sum(ys, inv, T, top_k, K, out, ldo, stream);
}

hipError_t launch_gated_mlp_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_gate_up,
                                 int64_t K, int64_t I, const float* alpha, const float* g2, void* h_codes,
                                 void* h_scales, float* h_amax, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (h_amax) hipLaunchKernelGGL(set_u32_kernel_moe, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(h_amax));
  const int32_t tiles = int32_t((M + gemm::BM - 1) / gemm::BM);
  // one workgroup fills a CU: the items run in rounds of one per CU; a last
  // round at most half full runs as 128-row halves
  const int64_t items = gemm::xcd_rows_grid(tiles, int32_t(I / 128));
  const int64_t cus = device_cu_count();
  const int64_t rest = items % cus;
  const int64_t n_big = (items > cus && rest > 0 && 2 * rest <= cus) ? items - rest : items;
  hipLaunchKernelGGL(gated_mlp_kernel, dim3(uint32_t(n_big + 2 * (items - n_big))), dim3(gemm::kThreads), 0, stream,
                     static_cast<const uint8_t*>(a_codes), static_cast<const uint8_t*>(a_scales), int32_t(K),
                     int32_t(M), static_cast<const uint8_t*>(w_gate_up), int32_t(I), alpha, g2,
                     static_cast<uint8_t*>(h_codes), static_cast<uint8_t*>(h_scales),
                     reinterpret_cast<uint32_t*>(h_amax), int32_t(n_big));
  return hipGetLastError();
}

}  // namespace nvfp4
