// Block-scaled NVFP4 x NVFP4 GEMM main loop for gfx950, shared by the dense
// W4A4 linear and the two grouped GEMMs of the MoE expert layer.
//
// Computes, for a workgroup tile of 256 weight rows x BMT activation rows
// (BMT = 256, or 128 for tiles that would be mostly empty or for a final
// partial round),
//   acc[row][tok] = sum_k deq(W)[row, k] * deq(A)[tok, k]
// with deq(x) = e2m1(code) * E4M3(scale of its 16-k group).  Every such value
// has at most 6 significant bits and lies in [2^-10, 2688], so it is exact in
// fp16, the products are exact in fp32 and the MFMA (32x32x16 fp16, fp32
// accumulate) adds exact terms.  (gfx950's fp4 MFMA scales by powers of two
// per 32 k and cannot carry NVFP4's per-16 E4M3 scales.)
//
// Per 64-k step the workgroup dequantizes both operand tiles once into LDS
// (fp16, row-major, double-buffered): the weight tile from the tiled weight
// (the step's 64 k of a 16-row tile are groups 4b..4b+3 of its unit, 8 code
// bytes and one scale byte per (row, group)), the activation tile from the
// canonical [rows, K/2] codes and [rows, K/16] scales.  The loads come in
// pairs of steps (128 k): a weight item's 16 code bytes of both steps and its
// unit's 4 scale bytes, an activation piece's 16 code bytes per step and its
// row's 8 scale bytes of the pair, so every code load is a dwordx4 and no load
// is narrower than a dword pair.  A pair is loaded two steps before its first
// step is dequantized; one barrier per step.
// Waves are laid out 2 (weight rows) x 4 (activation rows); each owns 128 x
// BMT/4 outputs as 4 x BMT/128 MFMA tiles of 32 x 32 (the 32x32x16 shape runs at about
// 1.6 times the rate of 16x16x32 on gfx950).  Register i of lane l in tile
// (t, u) holds weight row row0(t) + 8*(i/4) + 4*(l/32) + i%4 for activation
// row 32u + l%32 of the wave's BMT/4; with kSwap (operands exchanged in the
// MFMA) it holds weight row row0(t) + l%32 for activation row 32u + 8*(i/4) +
// 4*(l/32) + i%4, so that a register's 32 lanes cover 32 consecutive outputs
// of one activation row.
#pragma once

#include "device.hpp"

namespace nvfp4 {
namespace gemm {

constexpr int BN = 256;  // weight rows per workgroup (16 tiles of 16)
constexpr int BM = 256;  // activation rows per workgroup
constexpr int BK = 64;   // k per step
constexpr int PITCH = BK + 8;  // fp16 per LDS row; the pad staggers rows across banks
constexpr int kThreads = 512;
constexpr int kUnitBytes = 2304;
constexpr int kLdsHalves = 2 * (BN + BM) * PITCH;  // both buffers of both operands

// Workgroup -> output tile, XCD-aware.  Workgroups are dispatched to the 8
// XCDs in turn (id % 8), and each XCD has its own L2.  So workgroup id goes to
// position id / 8 of XCD id % 8's contiguous share of the tile order, and the
// order walks groups of kGroupM activation-row blocks with the rows fastest:
// the workgroups an XCD runs at once cover a compact block of tiles whose
// operand panels they share through that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__host__ __device__ inline int32_t xcd_grid(int32_t total) { return (total + kXcds - 1) / kXcds * kXcds; }

// Tile L (0 <= L < nt*mt) of the grouped order -> (n, m).
__device__ __forceinline__ void grouped_tile(int32_t L, int32_t nt, int32_t mt, int32_t& n, int32_t& m) {
  const int32_t gsize = kGroupM * nt;
  const int32_t first = (L / gsize) * kGroupM;
  const int32_t gm = min(mt - first, kGroupM);
  const int32_t r = L % gsize;
  m = first + r % gm;
  n = r / gm;
}

// The first `count` tiles of the grouped order, dealt to the XCDs as above;
// false for the padding workgroups of xcd_grid(count).
__device__ __forceinline__ bool xcd_tile(int32_t id, int32_t nt, int32_t mt, int32_t count, int32_t& n, int32_t& m) {
  const int32_t per = (count + kXcds - 1) / kXcds;
  const int32_t L = (id % kXcds) * per + id / kXcds;
  if (L >= count) return false;
  grouped_tile(L, nt, mt, n, m);
  return true;
}

__device__ __forceinline__ bool xcd_tile(int32_t id, int32_t nt, int32_t mt, int32_t& n, int32_t& m) {
  const int32_t total = nt * mt;
  const int32_t per = (total + kXcds - 1) / kXcds;
  const int32_t L = (id % kXcds) * per + id / kXcds;
  if (L >= total) return false;
  const int32_t gsize = kGroupM * nt;
  const int32_t first = (L / gsize) * kGroupM;
  const int32_t gm = min(mt - first, kGroupM);
  const int32_t r = L % gsize;
  m = first + r % gm;
  n = r / gm;
  return true;
}

// Grouped GEMMs: workgroup -> (tile-table row y, output block n) with all
// `nb` blocks of a row on one XCD (they share the row's gathered activation
// panel through its L2) and rows dealt to the XCDs in turn, so the live rows
// of a partly filled table are spread evenly.  Grid: xcd_rows_grid(rows, nb).
__host__ __device__ inline int32_t xcd_rows_grid(int32_t rows, int32_t nb) {
  return (rows + kXcds - 1) / kXcds * kXcds * nb;
}

__device__ __forceinline__ void xcd_row_block(int32_t id, int32_t nb, int32_t& y, int32_t& n) {
  const int32_t local = id / kXcds;
  y = (local / nb) * kXcds + id % kXcds;
  n = local % nb;
}

template <int BMT>
struct AccT {
  f32x16_t v[4][BMT / 128];  // [wave 32-row weight tile t][32-row activation tile u]
};
using Acc = AccT<BM>;

// Staged (not yet dequantized) operand bytes of a pair of steps (2p, 2p+1)
// for this thread.
struct Stage {
  uint4 w[2];      // weight items j: 16 codes of step 2p (x, y) and of step 2p+1 (z, w)
  uint32_t ws[2];  // their unit's scale bytes (steps 0..3 of the unit, byte b = step b)
  uint4 a[2];      // activation: 32 codes of row tid/2, k 32*(tid&1) .. +32, of step 2p+h
  uint2 as;        // the row's 8 scale bytes of the pair (x: step 2p, y: step 2p+1)
};

// The operands are read with buffer loads: a descriptor (scalar registers)
// holds the base address, each thread keeps the byte offsets of its pieces
// that do not depend on the step (one VGPR each), and the step adds a uniform
// offset in a scalar register -- no per-load address arithmetic.  Offsets are
// 32-bit: the weight descriptor starts at the workgroup's first weight tile
// (wtile(lt) >= wtile(0) for every lt), the activation one at row 0, and the
// callers keep both spans below 4 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(0xFFFFFFFF), 0x00020000);
}

// Weight item i (0..1023) of a step = (local tile lt = i / 64, lane slot
// l = i % 64 = r + 16q): row 16*lt + r, group 4b + q of the step's unit, b =
// the step within the unit.
struct StageOffsets {
  uint32_t w[2];   // item's unit row start (relative to the descriptor) + 16*l
  uint32_t ws[2];  // the same + 2048 + 4*l (scale bytes)
  uint32_t a;      // activation codes of row tid/2, k 32*(tid&1)
  uint32_t as;     // its scale bytes (the row's)
};

template <typename WTile, typename ARow>
__device__ __forceinline__ StageOffsets stage_offsets(WTile wtile, ARow a_row, int32_t steps256, int32_t K) {
  const int tid = int(threadIdx.x);
  const int64_t t0 = wtile(0);
  StageOffsets o;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + kThreads * j;
    const int lt = i >> 6, l = i & 63;
    const uint32_t unit0 = uint32_t(wtile(lt) - t0) * uint32_t(steps256) * uint32_t(kUnitBytes);
    o.w[j] = unit0 + 16u * uint32_t(l);
    o.ws[j] = unit0 + 2048u + 4u * uint32_t(l);
  }
  const uint32_t arow = uint32_t(a_row(tid >> 1)), half = uint32_t(tid & 1);
  o.a = arow * uint32_t(K / 2) + 16u * half;
  o.as = arow * uint32_t(K / 16);
  return o;
}

struct StageSrc {
  __amdgpu_buffer_rsrc_t w, a, as;
};

// Loads of pair p: the unit of the pair's steps is p / 2 and its code chunk
// (steps 4(p/2) + 2c, + 1) is c = p % 2.
__device__ __forceinline__ Stage load_pair(const StageSrc& src, const StageOffsets& o, int32_t p) {
  const int32_t wu = (p >> 1) * kUnitBytes;
  const int32_t wc = wu + 1024 * (p & 1);
  Stage s;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.w, o.w[j], wc, 0);
    s.w[j] = make_uint4(v[0], v[1], v[2], v[3]);
    s.ws[j] = __builtin_amdgcn_raw_buffer_load_b32(src.w, o.ws[j], wu, 0);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.a, o.a, p * BK + h * (BK / 2), 0);
    s.a[h] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  const auto sv = __builtin_amdgcn_raw_buffer_load_b64(src.as, o.as, p * (2 * BK / 16), 0);
  s.as = make_uint2(sv[0], sv[1]);
  return s;
}

// Dequantizes part `part` (0..3) of step h (0, 1) of a staged pair with code
// chunk c into LDS: parts 0 and 1 are the thread's two weight items, parts 2
// and 3 the two 16-k groups of its activation piece.  Split in four so the
// work interleaves with the MFMAs.
template <int BMT>
__device__ __forceinline__ void store_part(const Stage& s, int c, int h, int part, _Float16* __restrict__ wbuf,
                                           _Float16* __restrict__ abuf) {
  const int tid = int(threadIdx.x);
  uint32_t v0[4], v1[4];
  if (part < 2) {
    const int i = tid + kThreads * part;
    const int lt = i >> 6, l = i & 63, r = l & 15, q = l >> 4;
    // the step's scale byte: step 2c + h of the unit
    const uint32_t S2 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(s.ws[part] >> (8 * (2 * c + h)), 0));
    dequant8_f16(h == 0 ? s.w[part].x : s.w[part].z, S2, v0);
    dequant8_f16(h == 0 ? s.w[part].y : s.w[part].w, S2, v1);
    uint4* d = reinterpret_cast<uint4*>(wbuf + (16 * lt + r) * PITCH + 16 * q);
    d[0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
    d[1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
  } else {
    const int g = part - 2;  // 16-k group of the thread's 32 k
    const int row = tid >> 1, half = tid & 1;
    // narrow tiles stage fewer activation rows: waves BMT/32.. have none (a
    // wave-uniform test, so it is a scalar branch)
    if (BMT < BM && __builtin_amdgcn_readfirstlane(tid >> 6) >= BMT / 32) return;
    // group 2 half + g of the step: byte 2 half + g of the step's scale dword
    const uint32_t sb = (h == 0 ? s.as.x : s.as.y) >> (8 * (2 * half + g));
    const uint32_t S2 = f32_to_f16x2_splat(__builtin_amdgcn_cvt_f32_fp8(sb, 0));
    const uint4& ca = s.a[h];
    dequant8_f16(g == 0 ? ca.x : ca.z, S2, v0);
    dequant8_f16(g == 0 ? ca.y : ca.w, S2, v1);
    uint4* d = reinterpret_cast<uint4*>(abuf + row * PITCH + 32 * half + 16 * g);
    d[0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
    d[1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
  }
}

// MFMAs of the last 16-k block of a step that are issued after the barrier
// that ends the step, right after the next step's first LDS reads: every
// wave leaves the barrier at once and waits for those reads, and the held
// MFMAs keep the matrix pipe busy meanwhile.  Their operands are registers,
// and each accumulator still receives its products in k order, so the
// results are the same bits.  Holding the last weight tile (2 MFMAs per wave
// at 256 activation rows) took the GEMM at N = 8704, K = 5120 from 108.5 to
// 103.4 us (M = 1024) and from 591 to 577 us (M = 8192); holding two was no
// better.
constexpr int kHoldT = 1;  // wave 32-row weight tiles t = 4 - kHoldT .. 3 are held

template <int BMT>
struct HeldT {
  f16x8_t a[kHoldT];
  f16x8_t b[BMT / 128];
};

template <bool kSwap, int BMT>
__device__ __forceinline__ void issue_held(AccT<BMT>& acc, const HeldT<BMT>& held) {
#pragma unroll
  for (int i = 0; i < kHoldT; ++i)
#pragma unroll
    for (int u = 0; u < BMT / 128; ++u) {
      const int t = 4 - kHoldT + i;
      acc.v[t][u] = kSwap ? __builtin_amdgcn_mfma_f32_32x32x16_f16(held.b[u], held.a[i], acc.v[t][u], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_f16(held.a[i], held.b[u], acc.v[t][u], 0, 0, 0);
    }
}

// acc += W tile x A tile over one step (four 16-k MFMA blocks); after block
// kk, part kk of the next step (step nh of the staged pair `next`, code chunk
// nc) is dequantized into the other LDS buffer, so the VALU work runs under the
// MFMAs.  (After the last step the staged pair is a re-read of the last one
// and lands in a buffer nobody reads.)  The held MFMAs of the previous step
// are issued first (zero operands before the first step add nothing), and
// this step's are left in `held`.
// wave_row0(t) = first LDS weight row of the wave's 32-row tile t.
template <bool kSwap, int BMT, typename WaveRow0>
__device__ __forceinline__ void mma_step(AccT<BMT>& acc, HeldT<BMT>& held, const _Float16* __restrict__ wbuf,
                                         const _Float16* __restrict__ abuf, WaveRow0 wave_row0, int wm, int lane,
                                         const Stage& next, int nc, int nh, _Float16* __restrict__ wnext,
                                         _Float16* __restrict__ anext) {
  const int r = lane & 31, h = lane >> 5;
  // operands of block kk + 1 are read from LDS while the MFMAs of block kk run
  constexpr int U = BMT / 128;
  f16x8_t A[2][4], B[2][U];
  auto read = [&](int kk, int slot) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      B[slot][u] = *reinterpret_cast<const f16x8_t*>(abuf + (wm * (BMT / 4) + 32 * u + r) * PITCH + 16 * kk + 8 * h);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      A[slot][t] = *reinterpret_cast<const f16x8_t*>(wbuf + (wave_row0(t) + r) * PITCH + 16 * kk + 8 * h);
  };
  read(0, 0);
  issue_held<kSwap, BMT>(acc, held);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int cur = kk & 1;
    const bool last = kk + 1 == BK / 16;
    if (!last) read(kk + 1, cur ^ 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (last && t >= 4 - kHoldT) continue;
        acc.v[t][u] = kSwap ? __builtin_amdgcn_mfma_f32_32x32x16_f16(B[cur][u], A[cur][t], acc.v[t][u], 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_32x32x16_f16(A[cur][t], B[cur][u], acc.v[t][u], 0, 0, 0);
      }
    store_part<BMT>(next, nc, nh, kk, wnext, anext);
    // One MFMA, then a few VALU instructions of the staged dequant (and the
    // next block's LDS reads): the wave keeps its MFMA pipe busy while its own
    // VALU work issues in the MFMAs' shadow, instead of issuing the MFMAs
    // back to back and the VALU work after them.
    constexpr int kLastMfma = (4 - kHoldT) * U;
#pragma unroll
    for (int i = 0; i < (last ? kLastMfma : 4 * U); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // LDS write
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < kHoldT; ++i) held.a[i] = A[1][4 - kHoldT + i];
#pragma unroll
  for (int u = 0; u < U; ++u) held.b[u] = B[1][u];
}

// The K loop of one workgroup tile over the 128-k pairs [p_begin, p_begin +
// p_count) of K (K % 256 == 0; p_begin and p_count even, so the range is
// whole 256-k units; by default all of K).
//   a_row(i)    global activation row of tile row i (0..255): always a valid row
//               (rows BMT..255 are loaded but not used by a narrow tile)
//   wtile(lt)   tile index in the tiled weight of LDS weight tile lt (0..15): always valid
//   wave_row0(t) first LDS weight row of the calling wave's 32-row tile t (0..3)
template <bool kSwap = false, int BMT = BM, typename ARow, typename WTile, typename WaveRow0>
__device__ __forceinline__ void mainloop(AccT<BMT>& acc, _Float16* __restrict__ lds, const uint8_t* __restrict__ a_codes,
                                         const uint8_t* __restrict__ a_scales, ARow a_row,
                                         const uint8_t* __restrict__ wt, WTile wtile, WaveRow0 wave_row0, int32_t K,
                                         int32_t p_begin = 0, int32_t p_count = -1) {
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const int32_t pairs = p_count < 0 ? K / (2 * BK) : p_count, steps256 = K / 256;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < BMT / 128; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc.v[t][u][i] = 0.f;
  HeldT<BMT> held;
#pragma unroll
  for (int i = 0; i < kHoldT; ++i) held.a[i] = f16x8_t{};
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u) held.b[u] = f16x8_t{};
  const StageOffsets so = stage_offsets(wtile, a_row, steps256, K);
  StageSrc src;
  src.w = buffer_rsrc(wt + wtile(0) * steps256 * kUnitBytes);
  src.a = buffer_rsrc(a_codes);
  src.as = buffer_rsrc(a_scales);
  // buffer b of the weight tile at lds + b * BN * PITCH, of the activation
  // tile at lds + 2 * BN * PITCH + b * BMT * PITCH (offsets, so that the
  // compiler keeps every access in the LDS address space)
  _Float16* const abase = lds + 2 * BN * PITCH;
  _Float16* const w0 = lds;
  _Float16* const w1 = lds + BN * PITCH;
  _Float16* const a0 = abase;
  _Float16* const a1 = abase + BMT * PITCH;

  // Pairs alternate between the staging sets X and Y by name (the loop runs
  // two pairs per iteration), so no staged register is copied while its load
  // is in flight, and every iteration issues the same loads (past the last
  // pair they re-read it, unused): the compiler's wait counts then stay exact
  // around the loop.  A pair is loaded during the step two before the one
  // that dequantizes its first step, so its loads have two steps to land.
  // The loop has one exit, at its end (a mid-loop exit made the register
  // allocator move the accumulators through memory).
  Stage X = load_pair(src, so, p_begin);
  Stage Y = load_pair(src, so, p_begin + min(1, pairs - 1));
#pragma unroll
  for (int part = 0; part < 4; ++part) store_part<BMT>(X, 0, 0, part, w0, a0);
  __syncthreads();
  for (int32_t p = 0; p < pairs; p += 2) {
    // step 2p (buffer 0); step 2p+1, the second of X, -> buffer 1
    mma_step<kSwap, BMT>(acc, held, w0, a0, wave_row0, wm, lane, X, p & 1, 1, w1, a1);
    __syncthreads();
    // step 2p+1 (buffer 1); step 2p+2, the first of Y, -> buffer 0; X <- pair p+2
    X = load_pair(src, so, p_begin + min(p + 2, pairs - 1));
    mma_step<kSwap, BMT>(acc, held, w1, a1, wave_row0, wm, lane, Y, (p + 1) & 1, 0, w0, a0);
    __syncthreads();
    // step 2p+2 (buffer 0); step 2p+3, the second of Y, -> buffer 1
    mma_step<kSwap, BMT>(acc, held, w0, a0, wave_row0, wm, lane, Y, (p + 1) & 1, 1, w1, a1);
    __syncthreads();
    // step 2p+3 (buffer 1); step 2p+4, the first of X, -> buffer 0; Y <- pair p+3
    Y = load_pair(src, so, p_begin + min(p + 3, pairs - 1));
    mma_step<kSwap, BMT>(acc, held, w1, a1, wave_row0, wm, lane, X, p & 1, 0, w0, a0);
    __syncthreads();
  }
  issue_held<kSwap, BMT>(acc, held);
}

// Writes the bf16 tile out[m][n] (activation row m, weight row n) of the
// workgroup through LDS so that global stores are whole 16-byte pieces of
// output rows.  chunk(t, u, g) = the output values of accumulator registers
// 4g .. 4g+3 of wave tile (t, u) (a float4); rows beyond M and columns beyond
// N are not written.
// Needs out and ldo*2 aligned to 16 bytes and n0 % 8 == 0 (else a direct store).
template <int BMT = BM, typename Chunk>
__device__ __forceinline__ void store_tile_lds(_Float16* __restrict__ lds, Chunk chunk, uint16_t* __restrict__ out,
                                               int64_t ldo, int32_t m0, int32_t M, int32_t n0, int32_t N) {
  constexpr int OP = BN + 8;  // bf16 per LDS output row
  uint16_t* t16 = reinterpret_cast<uint16_t*>(lds);
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1, h = lane >> 5;
#pragma unroll
  for (int u = 0; u < BMT / 128; ++u) {
    const int mloc = wm * (BMT / 4) + 32 * u + (lane & 31);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nloc = 128 * wn + 32 * t + 8 * g + 4 * h;
        const float4 v = chunk(t, u, g);
        *reinterpret_cast<uint2*>(t16 + mloc * OP + nloc) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      }
  }
  __syncthreads();
  // BMT rows x 32 pieces of 8 bf16
  for (int e = int(threadIdx.x); e < BMT * (BN / 8); e += kThreads) {
    const int mloc = e >> 5, piece = e & 31;
    const int32_t m = m0 + mloc, n = n0 + 8 * piece;
    if (m >= M || n >= N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(t16 + mloc * OP + 8 * piece);
    uint16_t* dst = out + int64_t(m) * ldo + n;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if (n + 8 <= N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (n + i < N) dst[i] = uint16_t(w[i >> 1] >> (16 * (i & 1)));
    }
  }
}

}  // namespace gemm
}  // namespace nvfp4
