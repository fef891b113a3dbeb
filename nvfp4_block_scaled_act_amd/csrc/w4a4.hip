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
// A batch of at most 128 rows runs on its own kernel (skinny::kernel): each
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
// A batch of at most 128 rows (M <= 32 G, G = 1, 2 or 4 groups of 32 rows).
// The 256 x 256 tile main loop would run its tiles mostly empty here and
// stage every weight tile through LDS for a handful of rows; instead each
// wave dequantizes its own weight rows straight into MFMA operand registers
// and only the small activation tile goes through LDS, shared by the
// workgroup's waves.  A workgroup is 8 waves x one tile of 32 weight rows =
// 256 rows, over all M rows (or a range of whole 256-k units: split K); two
// waves per SIMD, so one wave's dequant issues under the other's MFMAs.
//
// MFMA operand order.  32x32x16 fp16: lane (r, h) (r = lane % 32, h = lane /
// 32) supplies 8 consecutive k-slots 8h..8h+7 of row r.  The contraction does
// not care which k a slot holds as long as both operands agree, so the 16
// MFMAs j = 2J + e (J = 0..7, e = 0, 1) of a 256-k unit give slot 8h + x the
// k = 16 (2J + h) + 8e + x: a lane takes the groups of its parity h.  In the
// tiled weight those are the groups 4p + q with q = h and q = h + 2 of lane
// slots r' + 16h and r' + 16(h + 2) (r' = r % 16): four 16-byte code loads
// and two scale dwords per lane and unit, all whole, and every lane uses all
// it loads.  The activation tile sits in LDS in plain k order (fp16, one
// padded row per activation row), so the B operand is one 16-byte read.
// Every value is exact in fp16 and every product in fp32, as in the main loop.
//
// Pipeline per 256-k step (one barrier): the weights of D steps live in
// registers, and after a step's MFMAs the next step's activation tile is
// dequantized into the other LDS buffer (see the kernel's ring).
namespace skinny {

constexpr int kWaves = 8;               // two waves per SIMD: one's dequant runs under the other's MFMAs
constexpr int kThreads = 64 * kWaves;
constexpr int TW = 1;                    // 32-row weight tiles per wave
constexpr int kRows = 32 * TW * kWaves;  // weight rows per workgroup
constexpr int kMaxM = 32 * 4;            // activation rows: up to four groups of 32
constexpr int PITCH = 256 + 8;           // fp16 per LDS activation row (the pad staggers rows across banks)

template <int G>
constexpr int lds_halves() {
  return 2 * 32 * G * PITCH;
}

struct WTileRegs {  // one lane's bytes of a 32-row tile's 256-k unit
  uint4 q[4];       // q = h groups p = 0,1 | p = 2,3; q = h + 2 groups p = 0,1 | p = 2,3
  uint32_t sc[2];   // scale bytes of the q = h groups (byte p), of the q = h + 2 groups
};
struct WRegs {
  WTileRegs t[TW];
};

// Activation pieces (32 codes of one row: 256 G per step) per thread; with
// fewer pieces than threads the waves past them stage none (a wave-uniform
// test).
template <int G>
constexpr int pieces_per_thread() {
  return (256 * G + kThreads - 1) / kThreads;
}

template <int G>
struct ARegs {      // a thread's activation pieces of one 256-k step
  uint4 c[pieces_per_thread<G>()];     // 32 codes: groups 2 pc, 2 pc + 1 of the step
  uint32_t s[pieces_per_thread<G>()];  // the dword holding their two scale bytes
};

struct Offsets {
  uint32_t w[TW];   // weight codes of lane slot r' + 16 h (relative to the descriptor)
  uint32_t ws[TW];  // its scale bytes
};

template <int G>
struct AOffsets {
  uint32_t c[pieces_per_thread<G>()], s[pieces_per_thread<G>()];
  int32_t lds[pieces_per_thread<G>()];    // fp16 offset of the piece in an LDS buffer
  int32_t shift[pieces_per_thread<G>()];  // bit offset of the piece's two scale bytes in the dword
};

template <int G>
__device__ __forceinline__ bool has_piece(int i) {
  return 256 * G >= kThreads * (i + 1) || __builtin_amdgcn_readfirstlane(int(threadIdx.x)) + kThreads * i < 256 * G;
}

__device__ __forceinline__ WRegs load_w(__amdgpu_buffer_rsrc_t rsrc, const Offsets& o, int32_t unit) {
  const int32_t so = unit * gemm::kUnitBytes;
  WRegs w;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    // lane slot r' + 16 (h + 2) is 32 slots on: 512 code bytes, 128 scale bytes
    const uint32_t offs[4] = {o.w[t], o.w[t] + 1024u, o.w[t] + 512u, o.w[t] + 1536u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, offs[i], so, 0);
      w.t[t].q[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    w.t[t].sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o.ws[t], so, 0);
    w.t[t].sc[1] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, o.ws[t] + 128u, so, 0);
  }
  return w;
}

template <int G>
__device__ __forceinline__ ARegs<G> load_a(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                           const AOffsets<G>& o, int32_t unit) {
  ARegs<G> a;
#pragma unroll
  for (int i = 0; i < pieces_per_thread<G>(); ++i) {
    if (!has_piece<G>(i)) {
      a.c[i] = make_uint4(0, 0, 0, 0);
      a.s[i] = 0;
      continue;
    }
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, o.c[i], unit * 128, 0);
    a.c[i] = make_uint4(v[0], v[1], v[2], v[3]);
    a.s[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.s[i], unit * 16, 0);
  }
  return a;
}

// Dequantizes the thread's pieces into LDS buffer buf (fp16, k order).
template <int G>
__device__ __forceinline__ void store_a(const ARegs<G>& a, const AOffsets<G>& o, _Float16* __restrict__ buf) {
#pragma unroll
  for (int i = 0; i < pieces_per_thread<G>(); ++i) {
    if (!has_piece<G>(i)) continue;
    const uint32_t sb = a.s[i] >> o.shift[i];
    const uint32_t S0 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(sb, 0));
    const uint32_t S1 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(sb, 1));
    uint32_t v[4][4];
    dequant8_f16(a.c[i].x, S0, v[0]);
    dequant8_f16(a.c[i].y, S0, v[1]);
    dequant8_f16(a.c[i].z, S1, v[2]);
    dequant8_f16(a.c[i].w, S1, v[3]);
    uint4* d = reinterpret_cast<uint4*>(buf + o.lds[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]);
  }
}

// Part `part` of store_a (8 codes of piece part / 4, dword part % 4), so the
// staging can be spread over a step's MFMA blocks.
template <int G>
constexpr int store_parts() {
  return 4 * pieces_per_thread<G>();
}

template <int G>
__device__ __forceinline__ void store_part(const ARegs<G>& a, const AOffsets<G>& o, _Float16* __restrict__ buf,
                                           int part) {
  const int i = part >> 2, q = part & 3;
  if (!has_piece<G>(i)) return;
  // groups 2 pc (dwords 0, 1) and 2 pc + 1 (dwords 2, 3) of the piece
  const uint32_t S = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8((a.s[i] >> o.shift[i]) >> (8 * (q >> 1)), 0));
  const uint32_t c[4] = {a.c[i].x, a.c[i].y, a.c[i].z, a.c[i].w};
  uint32_t v[4];
  dequant8_f16(c[q], S, v);
  *reinterpret_cast<uint4*>(buf + o.lds[i] + 8 * q) = make_uint4(v[0], v[1], v[2], v[3]);
}

// acc[t][g] += weight tile t x activation rows 32g.. over one 256-k step.
// Register i of lane l in acc[t][g] holds activation row 32g + 8(i/4) +
// 4(l/32) + i%4 and weight row 32t + l%32 of the wave's 64 (the activations
// are the MFMA's first operand, so a register's 32 lanes are 32 consecutive
// outputs of one activation row).  Software-pipelined by one MFMA block:
// the LDS reads and the weight dequant of block j + 1 are issued while the
// MFMAs of block j run, so neither the LDS latency nor the VALU work sits
// between two blocks' MFMAs.
template <int G>
__device__ __forceinline__ void read_b(f16x8_t (&B)[G], const _Float16* __restrict__ brow, int j) {
#pragma unroll
  for (int g = 0; g < G; ++g)
    B[g] = *reinterpret_cast<const f16x8_t*>(brow + 32 * g * PITCH + 32 * (j >> 1) + 8 * (j & 1));
}

// Weight operand of block j = 2J + e for tile t: codes of group 2J + h, half e.
__device__ __forceinline__ f16x8_t weight_a(const WTileRegs& w, int j) {
  const int J = j >> 1, e = j & 1;
  const uint32_t S2 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(w.sc[J & 1] >> (8 * (J >> 1)), 0));
  const uint4& q = w.q[(J & 1) * 2 + (J >> 2)];
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  uint32_t a[4];
  dequant8_f16(qw[((J >> 1) & 1) * 2 + e], S2, a);
  return __builtin_bit_cast(f16x8_t, make_uint4(a[0], a[1], a[2], a[3]));
}

// The next step's activation tile (codes `an`) is dequantized into nbuf in
// parts spread over the blocks, between their MFMAs.
template <int G>
__device__ __forceinline__ void step(f32x16_t (&acc)[TW][G], const WRegs& w, const _Float16* __restrict__ abuf,
                                     int lane, const ARegs<G>& an, const AOffsets<G>& ao,
                                     _Float16* __restrict__ nbuf) {
  const _Float16* brow = abuf + (lane & 31) * PITCH + 16 * (lane >> 5);
  f16x8_t B[2][G], A[2][TW];
  read_b<G>(B[0], brow, 0);
#pragma unroll
  for (int t = 0; t < TW; ++t) A[0][t] = weight_a(w.t[t], 0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int cur = j & 1;
    if (j < 15) read_b<G>(B[cur ^ 1], brow, j + 1);
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[t][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(B[cur][g], A[cur][t], acc[t][g], 0, 0, 0);
    if (j < 15) {
#pragma unroll
      for (int t = 0; t < TW; ++t) A[cur ^ 1][t] = weight_a(w.t[t], j + 1);
    }
    constexpr int every = 16 / store_parts<G>();
    if (j % every == every - 1) store_part<G>(an, ao, nbuf, j / every);
  }
}

// Workgroup id -> (row block blk = id % nblocks, K range s = id / nblocks).
// splits == 1: out[m][n] = bf16(alpha * acc); else the unscaled fp32 partial
// of range s at partials + s * M * N, row-major [M, N].
// D = steps of weights (and activation codes) held in registers: as deep as
// the register file allows at G groups of 32 rows.
template <int G, int D = (G == 4 ? 3 : 4)>
__global__ __launch_bounds__(kThreads) void kernel(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                                   int32_t M, const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                   const float* __restrict__ alpha_p, uint16_t* __restrict__ out,
                                                   int64_t ldo, float* __restrict__ partials, int32_t splits,
                                                   int32_t nblocks) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[lds_halves<G>()];
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int32_t id = int32_t(blockIdx.x);
  const int32_t blk = id % nblocks, s = id / nblocks;
  const int32_t units = K / 256;
  const int32_t u0 = int32_t(int64_t(s) * units / splits), u1 = int32_t(int64_t(s + 1) * units / splits);
  const int32_t nu = u1 - u0;
  const int32_t tiles16 = (N + 15) / 16, first16 = blk * (kRows / 16);

  // weight: the workgroup's rows start the descriptor; lane slot r' + 16h
  const __amdgpu_buffer_rsrc_t rw =
      gemm::buffer_rsrc(wt + int64_t(first16) * units * gemm::kUnitBytes);
  Offsets o;
  {
    const int r = lane & 31, lp = (r & 15) + 16 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int32_t t16 = min(first16 + 2 * (TW * wave + t) + (r >> 4), tiles16 - 1);
      const uint32_t base = uint32_t(t16 - first16) * uint32_t(units) * uint32_t(gemm::kUnitBytes);
      o.w[t] = base + 16u * uint32_t(lp);
      o.ws[t] = base + 2048u + 4u * uint32_t(lp);
    }
  }
  // Activation pieces: piece P = tid + kThreads i; each run of 64 pieces
  // covers 8 rows x the 8 pieces of a step (whole 128-byte lines of codes),
  // and each 8 neighbouring lanes 4 rows x 2 pieces, whose LDS rows (528
  // bytes apart) and pieces (64 bytes) put their 16-byte writes in 8
  // different bank groups.  (One row per lane had made every load
  // instruction touch 64 lines: at 64 rows that staging cost as much as the
  // MFMAs.)
  const __amdgpu_buffer_rsrc_t rac = gemm::buffer_rsrc(ac), ras = gemm::buffer_rsrc(as);
  AOffsets<G> ao;
#pragma unroll
  for (int i = 0; i < pieces_per_thread<G>(); ++i) {
    const int P = min(tid + kThreads * i, 256 * G - 1), l = P & 63;
    const int row = 8 * (P >> 6) + 4 * (l >> 5) + ((l >> 1) & 3), pc = 2 * ((l >> 3) & 3) + (l & 1);
    const uint32_t arow = uint32_t(min(row, M - 1));
    ao.c[i] = arow * uint32_t(K / 2) + 16u * uint32_t(pc);
    ao.s[i] = arow * uint32_t(K / 16) + 4u * uint32_t(pc >> 1);
    ao.shift[i] = 16 * (pc & 1);
    ao.lds[i] = row * PITCH + 32 * pc;
  }
  _Float16* const buf0 = lds;
  _Float16* const buf1 = lds + 32 * G * PITCH;

  f32x16_t acc[TW][G];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][g][i] = 0.f;

  // Ring of D stages: step st uses weights W[st % D] and stages the
  // activation codes A[(st + 1) % D] of the next step during its MFMAs; both
  // are loaded D steps ahead, the activations first: loads complete in issue
  // order, so waiting for the codes of step st + 1 waits for nothing later
  // than the weights of step st, which are in use.  Loads past the range
  // re-read its last unit (cache hits, never used).  The prologue's loads are
  // kept in program order (scheduling barriers), so the wait counts at the
  // loop head, which hold for the first entry as well as for the back edge,
  // are those of the steady state.
  auto unit = [&](int32_t i) { return u0 + min(i, nu - 1); };
  ARegs<G> A[D];
  WRegs W[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    A[d] = load_a<G>(rac, ras, ao, unit(d));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    W[d] = load_w(rw, o, unit(d));
    __builtin_amdgcn_sched_barrier(0);
  }
  store_a<G>(A[0], ao, buf0);
  __syncthreads();
  for (int32_t i = 0; i < nu; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int32_t st = i + d;
      if (st < nu)
        step<G>(acc, W[d], (st & 1) ? buf1 : buf0, lane, A[(d + 1) % D], ao, (st & 1) ? buf0 : buf1);
      A[d] = load_a<G>(rac, ras, ao, unit(st + D));
      W[d] = load_w(rw, o, unit(st + D));
      __syncthreads();
    }
  }

  const int h = lane >> 5;
  const int32_t n = blk * kRows + 32 * TW * wave + (lane & 31);
  if (splits == 1) {
    const float alpha = *alpha_p;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
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
    for (int t = 0; t < TW; ++t) {
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

}  // namespace skinny

}  // namespace

int w4a4_splits(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 256) return 1;
  const int64_t units = K / 256;
  const int64_t nt = (N + gemm::BN - 1) / gemm::BN, mt = (M + gemm::BM - 1) / gemm::BM;
  // one workgroup per 256-row column tile for a few rows (skinny::kernel)
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
      hipLaunchKernelGGL(skinny::kernel<1>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
                         alpha, O, ldo, part, splits, int32_t(nt));
    else if (M <= 64)
      hipLaunchKernelGGL(skinny::kernel<2>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
                         alpha, O, ldo, part, splits, int32_t(nt));
    else
      hipLaunchKernelGGL(skinny::kernel<4>, grid, block, 0, stream, AC, AS, int32_t(M), WT, int32_t(N), int32_t(K),
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
