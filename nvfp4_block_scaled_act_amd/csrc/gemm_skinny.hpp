// Few-rows NVFP4 x NVFP4 GEMM main loop for gfx950, shared by the dense
// W4A4 linear and the MoE expert GEMMs for tiles of at most 128 rows.
//
// For a tile of at most 128 activation rows (G = 1, 2 or 4 groups of 32 rows)
// the 256 x 256 tile main loop (gemm_w4a4.hpp) would run mostly empty and
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
// registers, and during a step's MFMAs the next step's activation tile is
// dequantized into the other LDS buffer (mainloop's ring).
#pragma once

#include "gemm_w4a4.hpp"

namespace nvfp4 {
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
  int32_t first;                          // the wave's first thread (wave-uniform)
};

template <int G>
__device__ __forceinline__ bool has_piece(const AOffsets<G>& o, int i) {
  return 256 * G >= kThreads * (i + 1) || o.first + kThreads * i < 256 * G;
}

// E4M3 scale bytes 2W and 2W + 1 of a dword as an fp16 pair, in one convert
// (exact: every E4M3 value is an fp16 value, and the convert's unit scale
// leaves them unchanged).
template <bool W>
__device__ __forceinline__ f16x2_t e4m3_pair_f16(uint32_t s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, W);
}

// Half H of a pair in both halves (the packed multiply reads it by operand
// select, so this costs no instruction).
template <int H>
__device__ __forceinline__ uint32_t splat_half(f16x2_t p) {
  return __builtin_bit_cast(uint32_t, __builtin_shufflevector(p, p, H, H));
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
    if (!has_piece<G>(o, i)) {
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
    if (!has_piece<G>(o, i)) continue;
    const f16x2_t sp = e4m3_pair_f16<false>(a.s[i] >> o.shift[i]);
    const uint32_t S0 = splat_half<0>(sp), S1 = splat_half<1>(sp);
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

// The scale pairs of the thread's pieces (groups 2 pc, 2 pc + 1), converted
// once per step for all its parts.
template <int G>
struct AScales {
  f16x2_t p[pieces_per_thread<G>()];
};

template <int G>
__device__ __forceinline__ AScales<G> a_scales(const ARegs<G>& a, const AOffsets<G>& o) {
  AScales<G> s;
#pragma unroll
  for (int i = 0; i < pieces_per_thread<G>(); ++i) s.p[i] = e4m3_pair_f16<false>(a.s[i] >> o.shift[i]);
  return s;
}

template <int G>
__device__ __forceinline__ void store_part(const ARegs<G>& a, const AScales<G>& as, const AOffsets<G>& o,
                                           _Float16* __restrict__ buf, int part) {
  const int i = part >> 2, q = part & 3;
  if (!has_piece<G>(o, i)) return;
  // groups 2 pc (dwords 0, 1) and 2 pc + 1 (dwords 2, 3) of the piece
  const uint32_t S = (q >> 1) ? splat_half<1>(as.p[i]) : splat_half<0>(as.p[i]);
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

// A tile's scale bytes of one step as fp16 pairs: p[d][W] holds bytes 2W,
// 2W + 1 of scale dword d.
struct WScales {
  f16x2_t p[2][2];
};

__device__ __forceinline__ WScales weight_scales(const WTileRegs& w) {
  WScales s;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    s.p[d][0] = e4m3_pair_f16<false>(w.sc[d]);
    s.p[d][1] = e4m3_pair_f16<true>(w.sc[d]);
  }
  return s;
}

// Weight operand of block j = 2J + e for tile t: codes of group 2J + h, half e
// (scale byte J / 2 of dword J % 2).
__device__ __forceinline__ f16x8_t weight_a(const WTileRegs& w, const WScales& ws, int j) {
  const int J = j >> 1, e = j & 1, p = J >> 1;
  const uint32_t S2 = (p & 1) ? splat_half<1>(ws.p[J & 1][p >> 1]) : splat_half<0>(ws.p[J & 1][p >> 1]);
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
  WScales ws[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) ws[t] = weight_scales(w.t[t]);
  const AScales<G> as = a_scales<G>(an, ao);
  f16x8_t B[2][G], A[2][TW];
  read_b<G>(B[0], brow, 0);
#pragma unroll
  for (int t = 0; t < TW; ++t) A[0][t] = weight_a(w.t[t], ws[t], 0);
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
      for (int t = 0; t < TW; ++t) A[cur ^ 1][t] = weight_a(w.t[t], ws[t], j + 1);
    }
    constexpr int every = 16 / store_parts<G>();
    if (j % every == every - 1) store_part<G>(an, as, ao, nbuf, j / every);
  }
}

// The K loop of one workgroup over the 256-k units [u0, u1) (u1 > u0):
// acc[t][g] = weight tile t of the wave x activation rows 32g.. (layout as in
// step()).
//   a_row(i)    activation row of tile row i (0 <= i < 32 G): always a valid
//               row (callers repeat the last one past their rows)
//   wtile16(j)  tiled-weight index of the workgroup's 16-row tile j (0..15),
//               non-decreasing in j and always valid: the weight descriptor
//               starts at wtile16(0), with 32-bit byte offsets from there
//   K           the reduction length (the activations' row length)
// lds holds lds_halves<G>() halves; the loop ends with a barrier, so the
// caller may reuse them at once.
template <int G, int D, typename ARow, typename WTile16>
__device__ __forceinline__ void mainloop(f32x16_t (&acc)[TW][G], _Float16* __restrict__ lds,
                                         const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, ARow a_row,
                                         const uint8_t* __restrict__ wt, WTile16 wtile16, int32_t K, int32_t u0,
                                         int32_t u1) {
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int32_t units = K / 256, nu = u1 - u0;

  // weight: lane slot r' + 16h of the wave's tiles
  const int64_t t0 = wtile16(0);
  const __amdgpu_buffer_rsrc_t rw = gemm::buffer_rsrc(wt + t0 * units * gemm::kUnitBytes);
  Offsets o;
  {
    const int r = lane & 31, lp = (r & 15) + 16 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int64_t t16 = wtile16(2 * (TW * wave + t) + (r >> 4));
      const uint32_t base = uint32_t(t16 - t0) * uint32_t(units) * uint32_t(gemm::kUnitBytes);
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
  ao.first = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
  for (int i = 0; i < pieces_per_thread<G>(); ++i) {
    const int P = min(tid + kThreads * i, 256 * G - 1), l = P & 63;
    const int row = 8 * (P >> 6) + 4 * (l >> 5) + ((l >> 1) & 3), pc = 2 * ((l >> 3) & 3) + (l & 1);
    const uint32_t arow = uint32_t(a_row(row));
    ao.c[i] = arow * uint32_t(K / 2) + 16u * uint32_t(pc);
    ao.s[i] = arow * uint32_t(K / 16) + 4u * uint32_t(pc >> 1);
    ao.shift[i] = 16 * (pc & 1);
    ao.lds[i] = row * PITCH + 32 * pc;
  }
  _Float16* const buf0 = lds;
  _Float16* const buf1 = lds + 32 * G * PITCH;

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
}

// D = steps of weights (and activation codes) held in registers: as deep as
// the register file allows at G groups of 32 rows.
template <int G>
constexpr int depth() {
  return G == 4 ? 3 : 4;
}

}  // namespace skinny
}  // namespace nvfp4
