// W4A16 NVFP4 linear for decode-sized M (M <= 64) on gfx950.
//
// Computes out[m, n] = bf16(alpha * sum_k a[m, k] * e2m1(c[n, k]) * E4M3(s[n, k/16]))
// with fp32 accumulation (FlashInfer PR #3597, Description: out = (a @
// dequant(b, b_sf).T) * alpha), on the weight re-tiled once by the prepare step.
//
// Arithmetic:
//  * swap-AB bf16 MFMA 16x16x32: 16 weight rows on the MFMA's row side, up to 16
//    tokens on its column side (token lanes >= M repeat token M-1; their output
//    columns are never stored);
//  * a 256-k step of a 16-row tile is one 2304-byte unit of the tiled weight;
//    a wave reads it with two dwordx4 code loads and one dword scale load per
//    lane, each instruction covering whole cache lines, and every lane then
//    holds the operands of its MFMA row: lane (r, q) owns the 16-k groups
//    4p + q (p = 0..3), so MFMA j = 2p + h multiplies codes k = 64p + 16q + 8h
//    + (0..7) of the step -- the same k the activation lane (c, q) reads;
//  * dequant: fp4 pair -> f32 pair (hardware convert, exact), times the E4M3
//    scale, packed to bf16 -- exact, since every e2m1 * E4M3 product fits bf16.
//
// The weight is read once from HBM.  Every 16-row tile needs all M x K
// activations (M/4.5 times the tile's weight bytes), and there are three
// schedules for them, each one launch with a fixed fp32 sum order
// (deterministic) and no workspace:
//  * split -- for weights with few row tiles: a workgroup owns one tile and its
//    `ksplit` waves split K, each reading its own activations through L1/L2;
//    the partial tiles are added through LDS in wave order.  This spreads a
//    small weight over enough waves to fill the GPU.  The fixed-step form
//    (at most 8 steps per wave) is fully unrolled so that the next step's
//    loads stay in flight under the current step's waits; its interleaved
//    variant gives wave w the steps w, w + waves, ... so the waves on a CU
//    read the same activation steps at a time.  With more than 4 token rows
//    the activation loads are issued in a cache-line-friendly lane order and
//    moved to their MFMA lanes by a cross-lane permute.
//  * shared -- for weights with many row tiles: a workgroup owns 8 tiles (16
//    on weights of at least 1.5 x 8 tiles per CU; one per wave) over all of K
//    and streams the activations through LDS in double-buffered chunks of `kc`
//    steps, so each chunk is read from L2 once per 8 or 16 tiles and from LDS
//    by every wave.
//  * dot -- up to 4 tokens, the split schedule's work split on the VALU
//    instead of the MFMA: each lane loads 4 activations per token and step
//    (no duplicates), the dot-product instruction broadcasts them across the
//    lane's row, and the dequant is one convert per code pair.
#include "device.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <atomic>

namespace nvfp4 {

namespace {

constexpr int kUnitBytes = 2304;
constexpr int kSharedTiles = 8;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Unit {
  uint4 c0, c1;
  uint32_t sc;
};

__device__ __forceinline__ Unit load_unit(const uint8_t* __restrict__ u, int lane) {
  Unit x;
  x.c0 = ld16_nt(u + 16 * lane);
  x.c1 = ld16_nt(u + 1024 + 16 * lane);
  x.sc = ld4_nt(u + 2048 + 4 * lane);
  return x;
}

// The same without the nontemporal hint (a cache-policy tactic, measured
// against the default: it slows the linear and the kernels after it).
__device__ __forceinline__ Unit load_unit_cached(const uint8_t* __restrict__ u, int lane) {
  Unit x;
  x.c0 = ld16(u + 16 * lane);
  x.c1 = ld16(u + 1024 + 16 * lane);
  x.sc = *reinterpret_cast<const uint32_t*>(u + 2048 + 4 * lane);
  return x;
}

// acc += dequant(codes of MFMAs 4*half .. 4*half+3) * b[0..3].
// A step that is not live (a re-read past the wave's last step) gets zero
// scales, so its products add nothing.
__device__ __forceinline__ void mma_half(const uint4& codes, uint32_t sc, int half, const uint4 (&b)[4],
                                         f32x4_t& acc, bool live = true) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  float S0 = half == 0 ? e4m3_to_f32<0>(sc) : e4m3_to_f32<2>(sc);
  float S1 = half == 0 ? e4m3_to_f32<1>(sc) : e4m3_to_f32<3>(sc);
  if (!live) S0 = S1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t av[4];
    dequant8_bf16(cw[i], i < 2 ? S0 : S1, av);
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(av[0], av[1], av[2], av[3]));
    const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b[i]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
  }
}

// Lane (c, qq) holds out[c][16 * tile + 4qq + i], i = 0..3.
__device__ __forceinline__ void store_tile(const f32x4_t& acc, float alpha, int lane, int32_t tile, int32_t M,
                                           int32_t N, uint16_t* __restrict__ out, int64_t ldo) {
  const int c = lane & 15, qq = lane >> 4;
  if (c >= M) return;
  uint16_t* orow = out + int64_t(c) * ldo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t n = 16 * tile + 4 * qq + i;
    if (n < N) orow[n] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * alpha));
  }
}

// The alpha operand lives in device memory (so that a captured call can take a
// new value).  Its load is issued with a kernel's first weight loads and
// awaited right after them, where its latency hides under theirs: waiting for
// it only in the epilogue would add a dependent memory round trip to the end
// of every (short) decode call.
__device__ __forceinline__ void settle(float& alpha) { asm volatile("" : "+s"(alpha)); }

// ------------------------------------------------------------------- split
// Activation operands of the 8 MFMAs of one 256-k step for lane (c, q): token
// row c's k = 64p + 16q + 8h + (0..7) for MFMA j = 2p + h.
struct StepB {
  uint4 v[8];
};

__device__ __forceinline__ StepB load_b(const uint16_t* __restrict__ astep, int q) {
  StepB b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b.v[j] = ld16(astep + 64 * (j >> 1) + 16 * q + 8 * (j & 1));
  return b;
}

// The same operands through a buffer resource whose lanes of token rows >= M
// point past its end: the load returns zeros there without reading, and
// those lanes' operand columns only make output columns that are never
// stored.  (The host keeps every real offset below 2^31.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const uint16_t* a) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a), short(0), int(0x7fffffff), 0x00020000);
}

// byte offset of the lane's row and 16-k piece, or past the end
__device__ __forceinline__ uint32_t act_off(int64_t lda, int32_t M, int row, int q) {
  return row < M ? uint32_t(row) * uint32_t(lda) * 2u + 32u * uint32_t(q) : 0x80000000u;
}

__device__ __forceinline__ StepB load_b_rows(__amdgpu_buffer_rsrc_t r, uint32_t off, int32_t st) {
  StepB b;
  const uint32_t o = off + uint32_t(st) * 512u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4_t v = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, o + 128u * (j >> 1) + 16u * (j & 1), 0, 0));
    b.v[j] = make_uint4(v.x, v.y, v.z, v.w);
  }
  return b;
}

// With several token rows, lane (c, q) of the MFMA layout puts 16 different
// rows in every group of 4 neighbouring lanes, and the texture unit then
// looks up 4 cache lines per group.  The permuted load has lane 4c + q read
// what lane c + 16q needs (4 neighbours, one row, one line); one LDS-crossbar
// permute per dword (no LDS storage) then moves it to its MFMA lane.
__device__ __forceinline__ uint4 to_mfma_lane(const uint4& v, int src_byte) {
  return make_uint4(uint32_t(__builtin_amdgcn_ds_bpermute(src_byte, int(v.x))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(src_byte, int(v.y))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(src_byte, int(v.z))),
                    uint32_t(__builtin_amdgcn_ds_bpermute(src_byte, int(v.w))));
}

__device__ __forceinline__ void mma_step(const Unit& u, const StepB& b, f32x4_t& acc, bool live = true) {
  const uint4 b0[4] = {b.v[0], b.v[1], b.v[2], b.v[3]};
  const uint4 b1[4] = {b.v[4], b.v[5], b.v[6], b.v[7]};
  mma_half(u.c0, u.sc, 0, b0, acc, live);
  mma_half(u.c1, u.sc, 1, b1, acc, live);
}

__device__ __forceinline__ void mma_step_perm(const Unit& u, const StepB& b, int src_byte, f32x4_t& acc, bool live) {
  const uint4 b0[4] = {to_mfma_lane(b.v[0], src_byte), to_mfma_lane(b.v[1], src_byte), to_mfma_lane(b.v[2], src_byte),
                       to_mfma_lane(b.v[3], src_byte)};
  mma_half(u.c0, u.sc, 0, b0, acc, live);
  const uint4 b1[4] = {to_mfma_lane(b.v[4], src_byte), to_mfma_lane(b.v[5], src_byte), to_mfma_lane(b.v[6], src_byte),
                       to_mfma_lane(b.v[7], src_byte)};
  mma_half(u.c1, u.sc, 1, b1, acc, live);
}

// Partial tiles of the waves added through LDS in wave order, then stored.
__device__ __forceinline__ void reduce_store(f32x4_t acc, float* red, int wave, int nwaves, int lane, int32_t tile,
                                             int32_t M, int32_t N, float alpha, uint16_t* __restrict__ out,
                                             int64_t ldo) {
  if (nwaves > 1) {
    *reinterpret_cast<f32x4_t*>(&red[(wave * 64 + lane) * 4]) = acc;
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < nwaves; ++w) acc += *reinterpret_cast<const f32x4_t*>(&red[(w * 64 + lane) * 4]);
  }
  store_tile(acc, alpha, lane, tile, M, N, out, ldo);
}

// Split with at most PER steps per wave, fully unrolled: step i+1's weight
// unit and activation operands are issued before step i is computed, in the
// order they are consumed (loads complete in issue order), and a scheduling
// barrier keeps the compiler from sinking them below step i's waits.  Steps
// past a wave's share re-read a valid step with zero scales.
// INTERLEAVE: wave w takes steps w, w + waves, w + 2*waves, ... instead of a
// contiguous run, so the waves of every workgroup on a CU read the same few
// activation steps at a time and share them in the L1 cache.
constexpr int kSplitMaxPer = 8;

// Up to R tiles per workgroup (R = 2 where a CU would otherwise hold two or
// more one-tile workgroups; R = 3 with one workgroup per CU holding 2 or 3
// tiles): each step's activation operands are loaded (and permuted) once and
// serve the workgroup's `count` tiles' weight units.
template <int R>
__device__ __forceinline__ void reduce_store_tiles(const f32x4_t (&acc)[R], float* red, int wave, int nwaves, int lane,
                                                   int32_t tile0, int32_t count, int32_t tiles, int32_t M, int32_t N,
                                                   float alpha, uint16_t* __restrict__ out, int64_t ldo) {
  if (nwaves == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < count && tile0 + r < tiles) store_tile(acc[r], alpha, lane, tile0 + r, M, N, out, ldo);
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) *reinterpret_cast<f32x4_t*>(&red[((wave * R + r) * 64 + lane) * 4]) = acc[r];
  __syncthreads();
  // nwaves >= R: wave r adds up tile r
  if (wave >= count || tile0 + wave >= tiles) return;
  f32x4_t sum = *reinterpret_cast<const f32x4_t*>(&red[(wave * 64 + lane) * 4]);
  for (int w = 1; w < nwaves; ++w) sum += *reinterpret_cast<const f32x4_t*>(&red[((w * R + wave) * 64 + lane) * 4]);
  store_tile(sum, alpha, lane, tile0 + wave, M, N, out, ldo);
}

template <int PER, bool INTERLEAVE, bool PERM, int R>
__global__ __launch_bounds__(R == 1 ? 1024 : 512) void w4a16_split_fixed_kernel(
    const uint16_t* __restrict__ a, int64_t lda, int32_t M, const uint8_t* __restrict__ wt, int32_t N, int32_t K,
    int32_t steps_per_wave, const float* __restrict__ alpha_p, uint16_t* __restrict__ out, int64_t ldo,
    int32_t full) {
  extern __shared__ float red[];  // [waves][R][64][4]
  const int lane = int(threadIdx.x & 63);
  const int wave = int(threadIdx.x >> 6);
  const int nwaves = int(blockDim.x >> 6);
  const int q = lane >> 4;
  const int32_t tiles = (N + 15) / 16;
  // workgroups [0, full) hold R consecutive tiles, the rest R - 1
  const int32_t wg = int32_t(blockIdx.x);
  const int32_t tile0 = wg * (R - 1) + min(wg, full);
  const int32_t count = R - 1 + (wg < full ? 1 : 0);
  const int32_t steps = K / 256;
  const int32_t s0 = INTERLEAVE ? wave : wave * steps_per_wave;
  const int32_t ds = INTERLEAVE ? nwaves : 1;
  const int32_t s1 = INTERLEAVE ? steps : min(steps, s0 + steps_per_wave);
  // the lane's load row and 16-k piece (PERM: lane 4c + q loads for MFMA lane c + 16q)
  const int lrow = PERM ? (lane >> 2) : (lane & 15), lq = PERM ? (lane & 3) : q;
  const int src_byte = 4 * (4 * (lane & 15) + q);
  const __amdgpu_buffer_rsrc_t arsrc = act_rsrc(a);
  const uint32_t aoff = act_off(lda, M, lrow, lq);
  // tiles past the last re-read the last tile; their results are not stored
  auto unit_at = [&](int r, int32_t st) {
    const int32_t t = min(tile0 + min(r, count - 1), tiles - 1);
    return load_unit(wt + (int64_t(t) * steps + min(st, steps - 1)) * kUnitBytes, lane);
  };
  auto b_at = [&](int32_t st) { return load_b_rows(arsrc, aoff, min(st, steps - 1)); };

  f32x4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Unit w[2][R];
  StepB b[2];
  float alpha = *alpha_p;
#pragma unroll
  for (int r = 0; r < R; ++r) w[0][r] = unit_at(r, s0);
  b[0] = b_at(s0);
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (i + 1 < PER) {
#pragma unroll
      for (int r = 0; r < R; ++r) w[(i + 1) & 1][r] = unit_at(r, s0 + (i + 1) * ds);
      b[(i + 1) & 1] = b_at(s0 + (i + 1) * ds);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool live = s0 + i * ds < s1;
    if (R == 1) {
      if (PERM)
        mma_step_perm(w[i & 1][0], b[i & 1], src_byte, acc[0], live);
      else
        mma_step(w[i & 1][0], b[i & 1], acc[0], live);
    } else {
      const StepB& bs = b[i & 1];
      uint4 b0[4], b1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = PERM ? to_mfma_lane(bs.v[j], src_byte) : bs.v[j];
        b1[j] = PERM ? to_mfma_lane(bs.v[4 + j], src_byte) : bs.v[4 + j];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (R < 3 || r < count) {  // (uniform) a two-tile workgroup of R = 3 skips its third
          mma_half(w[i & 1][r].c0, w[i & 1][r].sc, 0, b0, acc[r], live);
          mma_half(w[i & 1][r].c1, w[i & 1][r].sc, 1, b1, acc[r], live);
        }
      }
    }
  }
  reduce_store_tiles<R>(acc, red, wave, nwaves, lane, tile0, count, tiles, M, N, alpha, out, ldo);
}

// Each wave runs steps [s0, s1) of one tile.  Step s+1's weight unit and
// activation operands are loaded before step s is computed.  Loads complete in
// issue order, so they are issued in the order they are consumed, and every
// step issues the same loads (past s1 they re-read the last step, unused):
// the waits then only cover the step being computed and the next step's loads
// stay in flight.  Two register sets alternate by name (two steps per
// iteration), so nothing is copied while its load is outstanding.
__global__ __launch_bounds__(1024) void w4a16_split_kernel(
    const uint16_t* __restrict__ a, int64_t lda, int32_t M, const uint8_t* __restrict__ wt, int32_t N, int32_t K,
    int32_t steps_per_wave, const float* __restrict__ alpha_p, uint16_t* __restrict__ out, int64_t ldo) {
  extern __shared__ float red[];  // [waves][64][4]
  const int lane = int(threadIdx.x & 63);
  const int wave = int(threadIdx.x >> 6);
  const int nwaves = int(blockDim.x >> 6);
  const int q = lane >> 4;
  const int32_t tile = int32_t(blockIdx.x);
  const int32_t steps = K / 256;
  const int32_t s0 = wave * steps_per_wave;
  const int32_t s1 = min(steps, s0 + steps_per_wave);  // s0 < s1: the host sizes the block so
  const uint16_t* arow = a + int64_t(min(lane & 15, M - 1)) * lda;
  const uint8_t* wtile = wt + int64_t(tile) * steps * kUnitBytes;
  auto unit_at = [&](int32_t st) { return load_unit(wtile + int64_t(min(st, s1 - 1)) * kUnitBytes, lane); };
  auto b_at = [&](int32_t st) { return load_b(arow + 256 * int64_t(min(st, s1 - 1)), q); };

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float alpha = *alpha_p;
  Unit wa = unit_at(s0);
  StepB ba = b_at(s0);
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
  // (the scheduling barriers keep the compiler from sinking the next step's
  // loads below the current step's waits)
  for (int32_t s = s0;; s += 2) {
    const Unit wb = unit_at(s + 1);
    const StepB bb = b_at(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma_step(wa, ba, acc);
    if (s + 1 >= s1) break;
    wa = unit_at(s + 2);
    ba = b_at(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    mma_step(wb, bb, acc);
    if (s + 2 >= s1) break;
  }

  reduce_store(acc, red, wave, nwaves, lane, tile, M, N, alpha, out, ldo);
}

// ------------------------------------------------------------------ shared
// LDS holds two chunks of kc steps; a chunk is [kc steps][8 j][4 q][MP c]
// entries of 8 bf16: the M real token rows, with MP = M for one token group
// and M padded to the kernel's 16 MG rows above, so that the distance between
// the (j, q) blocks is a constant and the LDS reads of a step take immediate
// offsets.
//
// Thread e of the workgroup stages entry e (and e + threads, ...) of the
// chunk's real rows in token-row-fastest order, so the LDS writes of a wave
// are runs of M consecutive entries.  (With one token row per run of
// neighbouring threads their entries lay M apart and the writes of a wave all
// fell in one bank: about half of the kernel's LDS cycles were bank
// conflicts, and N = 62080, K = 5120 took 80/69/59 us at M = 64/48/32
// against 76/63/54 us without them.)  The global loads then take 16 bytes
// from each of up to 64 token rows per instruction; they hit L2.  Where an
// entry goes and what it loads is the same for every chunk, so it is computed
// once per thread (with the padded rows, about a sixth fewer VALU
// instructions at M = 64 and 2-6 % less time at M = 16 and 32).
struct SharedStage {
  int32_t dst[4];  // LDS entry in a chunk (kc * 32 * MP when the thread has none)
  int32_t src[4];  // token row c | (k offset in the chunk << 8)
};

__device__ __forceinline__ SharedStage shared_stage(int32_t M, int32_t MP, int32_t kc, int32_t tid, int32_t nthreads) {
  SharedStage st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t e = tid + i * nthreads;
    st.dst[i] = kc * 32 * MP;
    st.src[i] = 0;
    if (e < kc * 32 * M) {
      const int32_t rest = e / M, c = e - rest * M;  // rest = (s * 8 + j) * 4 + q
      const int32_t q = rest & 3, j = (rest >> 2) & 7, s = rest >> 5;
      st.dst[i] = rest * MP + c;
      // MFMA j = 2p + h of a step multiplies k = 64p + 16q + 8h + (0..7)
      st.src[i] = c | ((s * 256 + 64 * (j >> 1) + 16 * q + 8 * (j & 1)) << 8);
    }
  }
  return st;
}

// Loads of the chunk that starts at step s_begin and has ns steps.
__device__ __forceinline__ void shared_load(const uint16_t* __restrict__ a, int64_t lda, const SharedStage& st,
                                            int32_t MP, int32_t s_begin, int32_t ns, uint4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (st.dst[i] < ns * 32 * MP)
      v[i] = ld16(a + int64_t(st.src[i] & 255) * lda + int64_t(s_begin) * 256 + (st.src[i] >> 8));
}

__device__ __forceinline__ void shared_store(uint4* __restrict__ buf, const SharedStage& st, int32_t MP, int32_t ns,
                                             const uint4 (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (st.dst[i] < ns * 32 * MP) buf[st.dst[i]] = v[i];
}

// Lane (c, qq) of token group mg holds out[16 mg + c][16 * tile + 4qq + i].
__device__ __forceinline__ void store_tile_rows(const f32x4_t& acc, float alpha, int lane, int32_t tile, int32_t row0,
                                                int32_t M, int32_t N, uint16_t* __restrict__ out, int64_t ldo) {
  const int c = lane & 15, qq = lane >> 4;
  if (row0 + c >= M) return;
  uint16_t* orow = out + int64_t(row0 + c) * ldo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t n = 16 * tile + 4 * qq + i;
    if (n < N) orow[n] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * alpha));
  }
}

// MG token groups of 16 (M <= 16 MG): the codes of each MFMA operand are
// dequantized once and multiply the activation operands of every group, so
// the dequant work per weight does not grow with M.  TPW tiles (one per wave)
// per workgroup share each staged activation chunk.
template <int MG, int TPW>
__global__ __launch_bounds__(TPW * 64) void w4a16_shared_kernel(const uint16_t* __restrict__ a, int64_t lda, int32_t M,
                                                           const uint8_t* __restrict__ wt, int32_t N, int32_t K,
                                                           int32_t kc, const float* __restrict__ alpha_p,
                                                           uint16_t* __restrict__ out, int64_t ldo) {
  const int32_t MP = MG == 1 ? M : 16 * MG;  // LDS token rows per (step, j, q): a constant above one group
  extern __shared__ uint4 act[];  // two chunks of kc * 32 * MP entries
  const int lane = int(threadIdx.x & 63);
  const int wave = int(threadIdx.x >> 6);
  const int32_t tid = int32_t(threadIdx.x);
  const int32_t tiles = (N + 15) / 16;
  const int32_t steps = K / 256;
  const int32_t nch = (steps + kc - 1) / kc;
  const int32_t chunk_entries = kc * 32 * MP;
  const int32_t tile = int32_t(blockIdx.x) * TPW + wave;
  const bool has_tile = tile < tiles;
  // token row 16 mg + (lane % 16) of k sub-block lane / 16 (rows past M repeat
  // row M - 1; their outputs are not stored)
  int lds_lane[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) lds_lane[mg] = (lane >> 4) * MP + min(16 * mg + (lane & 15), M - 1);
  const uint8_t* wtile = wt + int64_t(has_tile ? tile : 0) * steps * kUnitBytes;

  // The weight units of the next kSharedDepth steps are in flight while a
  // step is computed: four named slots, each reloaded (unconditionally,
  // clamped to the last step) right after the step that consumed it.  Loads
  // complete in issue order, so the wait for a step's unit leaves the three
  // younger ones in flight; nothing is copied out of a slot whose load is
  // outstanding (that would wait for it, and for everything older).
  auto unit_at = [&](int32_t st) { return load_unit(wtile + int64_t(min(st, steps - 1)) * kUnitBytes, lane); };
  uint4 v[4];
  const SharedStage st = shared_stage(M, MP, kc, tid, TPW * 64);
  float alpha = *alpha_p;
  int32_t staged_ns = min(kc, steps);  // steps of the chunk in v
  shared_load(a, lda, st, MP, 0, staged_ns, v);
  Unit w0 = unit_at(0), w1 = unit_at(1), w2 = unit_at(2), w3 = unit_at(3);
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
  shared_store(act, st, MP, staged_ns, v);
  __syncthreads();

  f32x4_t acc[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) acc[mg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // step gs of chunk ch = gs / kc.  At a chunk's first step the chunk staged
  // during the previous one is written to its LDS buffer (every wave is past
  // the chunk before it, which used that buffer) and the next chunk's loads
  // are issued.
  auto step = [&](int32_t gs, const Unit& cur) {
    const int32_t ch = gs / kc, s = gs - ch * kc;
    if (s == 0 && ch > 0) {
      shared_store(act + (ch & 1) * chunk_entries, st, MP, staged_ns, v);
      __syncthreads();
    }
    if (s == 0 && ch + 1 < nch) {
      staged_ns = min(kc, steps - gs - kc);
      shared_load(a, lda, st, MP, gs + kc, staged_ns, v);
    }
    const uint4* lds_step = act + (ch & 1) * chunk_entries + s * 32 * MP;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (MG == 1) {
        uint4 bb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bb[i] = lds_step[(4 * half + i) * 4 * MP + lds_lane[0]];
        mma_half(half == 0 ? cur.c0 : cur.c1, cur.sc, half, bb, acc[0]);
      } else {
        const uint4 codes = half == 0 ? cur.c0 : cur.c1;
        const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
        const float S0 = half == 0 ? e4m3_to_f32<0>(cur.sc) : e4m3_to_f32<2>(cur.sc);
        const float S1 = half == 0 ? e4m3_to_f32<1>(cur.sc) : e4m3_to_f32<3>(cur.sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t av[4];
          dequant8_bf16(cw[i], i < 2 ? S0 : S1, av);
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(av[0], av[1], av[2], av[3]));
#pragma unroll
          for (int mg = 0; mg < MG; ++mg) {
            const bf16x8_t B = __builtin_bit_cast(bf16x8_t, lds_step[(4 * half + i) * 4 * MP + lds_lane[mg]]);
            acc[mg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[mg], 0, 0, 0);
          }
        }
      }
    }
  };
  for (int32_t gs = 0; gs < steps; gs += 4) {
    step(gs, w0);
    w0 = unit_at(gs + 4);
    __builtin_amdgcn_sched_barrier(0);
    if (gs + 1 < steps) step(gs + 1, w1);
    w1 = unit_at(gs + 5);
    __builtin_amdgcn_sched_barrier(0);
    if (gs + 2 < steps) step(gs + 2, w2);
    w2 = unit_at(gs + 6);
    __builtin_amdgcn_sched_barrier(0);
    if (gs + 3 < steps) step(gs + 3, w3);
    w3 = unit_at(gs + 7);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (has_tile) {
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) store_tile_rows(acc[mg], alpha, lane, tile, 16 * mg, M, N, out, ldo);
  }
}

// --------------------------------------------------------------------- dot
// A few tokens: the MFMA would spend most of its work on repeated token
// columns and the split kernel's texture unit on duplicate activation loads
// (eight 16-byte loads per wave and step whatever M is), so each lane computes
// plain dot products on the VALU.  Lane
// (r, q) of a unit holds row r's codes of the 16-k groups 4p + q (p = 0..3);
// its row of 16 lanes (q) needs the 64 activations k = 64p + 16q + 8h + i
// (h = 0..1, i = 0..7), and lane n of that row loads 4 of them (p = n / 4,
// h = (n / 2) % 2, i = 4 (n % 2) + 0..3) with one 8-byte load.  The
// dot-product instruction reads them from lane 4p + 2h + i / 4 of the row
// through its DPP row broadcast, so no lane holds a copy of another lane's
// activations.  The codes are converted to bf16 pairs (exact), each 16-k
// block's partial dot (fp32) is multiplied by the block scale as it is added
// to the lane's sum, the 4 lanes of a row are added (q order fixed), then the
// waves in wave order.

// The 32 products of a unit for one token: part[p] += dot(activation pair
// broadcast from lane 4p + s / 2 of the row (register x for even s, y for odd
// s), weight pair s of block p), s = 0..7.  A DPP instruction must not read a
// VGPR (any operand, the accumulator included) that a VALU instruction wrote
// in the two instructions before it, so the four blocks' chains are
// interleaved (each accumulator is read 3 instructions after its write) and a
// leading s_nop covers the operands written just before the block.
constexpr int kDotMaxM = 4;

template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL));
}

__device__ __forceinline__ void dot_unit(const uint2& x, const Unit& u, float (&part)[4]) {
  const uint32_t c[8] = {u.c0.x, u.c0.y, u.c0.z, u.c0.w, u.c1.x, u.c1.y, u.c1.z, u.c1.w};
  uint32_t w[32];  // w[8p + s]: pair s of block p (s < 4: low code dword, byte s; s >= 4: high dword, byte s - 4)
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    w[8 * pp + 0] = e2m1x2_to_bf16<0>(c[2 * pp]);
    w[8 * pp + 1] = e2m1x2_to_bf16<1>(c[2 * pp]);
    w[8 * pp + 2] = e2m1x2_to_bf16<2>(c[2 * pp]);
    w[8 * pp + 3] = e2m1x2_to_bf16<3>(c[2 * pp]);
    w[8 * pp + 4] = e2m1x2_to_bf16<0>(c[2 * pp + 1]);
    w[8 * pp + 5] = e2m1x2_to_bf16<1>(c[2 * pp + 1]);
    w[8 * pp + 6] = e2m1x2_to_bf16<2>(c[2 * pp + 1]);
    w[8 * pp + 7] = e2m1x2_to_bf16<3>(c[2 * pp + 1]);
  }
  asm volatile(
  "s_nop 1\n"
  "v_dot2c_f32_bf16_dpp %0, %4, %6 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %4, %14 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %4, %22 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %4, %30 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %5, %7 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %5, %15 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %5, %23 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %5, %31 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %4, %8 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %4, %16 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %4, %24 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %4, %32 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %5, %17 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %5, %25 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %5, %33 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %4, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %4, %26 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %4, %34 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %5, %11 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %5, %19 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %5, %27 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %5, %35 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %4, %12 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %4, %20 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %4, %28 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %4, %36 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %0, %5, %13 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %1, %5, %21 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %2, %5, %29 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
  "v_dot2c_f32_bf16_dpp %3, %5, %37 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
      : "+v"(part[0]), "+v"(part[1]), "+v"(part[2]), "+v"(part[3])
      : "v"(x.x), "v"(x.y), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]),
        "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]), "v"(w[16]),
        "v"(w[17]), "v"(w[18]), "v"(w[19]), "v"(w[20]), "v"(w[21]), "v"(w[22]), "v"(w[23]), "v"(w[24]), "v"(w[25]),
        "v"(w[26]), "v"(w[27]), "v"(w[28]), "v"(w[29]), "v"(w[30]), "v"(w[31]));
}

// acc[m] += sum over the lane's 64 k of the unit of token m: the 16-k blocks'
// partial dots times their block scales.
template <int MT>
__device__ __forceinline__ void dot_step(const Unit& u, const uint2 (&x)[MT], float (&acc)[MT]) {
  const float S[4] = {e4m3_to_f32<0>(u.sc), e4m3_to_f32<1>(u.sc), e4m3_to_f32<2>(u.sc), e4m3_to_f32<3>(u.sc)};
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    dot_unit(x[m], u, part);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) acc[m] = __builtin_fmaf(S[pp], part[pp], acc[m]);
  }
}

// Wave w takes steps w, w + waves, ... (PER of them; the ones past K are
// skipped) of the workgroup's tile, with the units and activations of two
// steps in flight while one is computed.
template <int PER, int MT, int CP>
__global__ __launch_bounds__(1024) void w4a16_dot_kernel(
    const uint16_t* __restrict__ a, int64_t lda, int32_t M, const uint8_t* __restrict__ wt, int32_t N, int32_t K,
    const float* __restrict__ alpha_p, uint16_t* __restrict__ out, int64_t ldo) {
  extern __shared__ float dot_red[];  // [16][MT][16]: a slot per possible wave
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6), nwaves = int(blockDim.x >> 6);
  const int q = lane >> 4, n = lane & 15;
  const int32_t tile = int32_t(blockIdx.x), steps = K / 256;
  const uint8_t* wtile = wt + int64_t(tile) * steps * kUnitBytes;
  const int koff = 64 * (n >> 2) + 16 * q + 8 * ((n >> 1) & 1) + 4 * (n & 1);
  const uint16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) arow[m] = a + int64_t(min(m, M - 1)) * lda + koff;
  // CP: the cache policy of the loads (0 the default; 1 weights without the
  // nontemporal hint; 2 activations with it)
  auto unit_at = [&](int32_t st) {
    const uint8_t* u = wtile + int64_t(min(st, steps - 1)) * kUnitBytes;
    return CP == 1 ? load_unit_cached(u, lane) : load_unit(u, lane);
  };
  auto act_at = [&](int32_t st, uint2 (&x)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint16_t* p = arow[m] + 256 * int64_t(min(st, steps - 1));
      if (CP == 2) {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        x[m] = make_uint2(v.x, v.y);
      } else {
        x[m] = *reinterpret_cast<const uint2*>(p);
      }
    }
  };

  float alpha = *alpha_p;
  Unit w[2];
  uint2 x[2][MT];
  act_at(wave, x[0]);
  w[0] = unit_at(wave);
  if (PER > 1) {
    act_at(wave + nwaves, x[1]);
    w[1] = unit_at(wave + nwaves);
  }
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (wave + i * nwaves < steps) dot_step<MT>(w[i & 1], x[i & 1], acc);
    if (i + 2 < PER) {
      act_at(wave + (i + 2) * nwaves, x[i & 1]);
      w[i & 1] = unit_at(wave + (i + 2) * nwaves);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the row's 4 lanes (q), then the waves in order
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc[m] += __shfl_xor(acc[m], 16, 64);
    acc[m] += __shfl_xor(acc[m], 32, 64);
  }
  if (nwaves > 1) {
    if (q == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) dot_red[(wave * MT + m) * 16 + n] = acc[m];
    }
    __syncthreads();
    if (wave != 0) return;
    // in wave order, from every slot read at once (the ones past nwaves are
    // read and dropped)
    float v[16][MT];
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int m = 0; m < MT; ++m) v[k][m] = dot_red[(k * MT + m) * 16 + n];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[m] = v[0][m];
#pragma unroll
      for (int k = 1; k < 16; ++k)
        if (k < nwaves) acc[m] += v[k][m];
    }
  }
  const int32_t row = 16 * tile + n;
  if (q == 0 && row < N) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) out[int64_t(m) * ldo + row] = __builtin_bit_cast(uint16_t, (__bf16)(acc[m] * alpha));
  }
}

// ---------------------------------------------------------------- grouped
// W4A16 on the experts of an MoE layer for decode-sized batches (the W4A16
// side of the layer's tokens-per-expert dispatch, FreeToken PR #736,
// Changes).  The align step cuts each expert's pairs into entries of up to 16
// (MoeTile); one workgroup computes one 16-row output tile of one entry, its
// waves taking interleaved 256-k steps, and the activation rows of a lane's
// token column are gathered by slot (x by token for gate_up, h by slot for
// down).  Lanes past the entry's pairs read nothing (out-of-range buffer
// offsets) and their columns are not stored.
//   GATED (gate_up): the workgroup computes gate tile t and up tile I/16 + t
//     of the expert (each step's activation operands serve both) and stores
//     h = bf16(SiLU(z_g) * z_u), z = alpha_e * acc, by slot;
//   else (down): it stores the routing-weighted y = w * (alpha_e * acc) in
//     fp32 by slot for the route sum.
// An entry of one or two pairs: the dot schedule's products on the VALU (each
// lane loads 4 activations per token and step, the dot-product instruction
// broadcasts them across the row; see the dot section), for the R tiles of
// the workgroup at once.
template <int PER, bool GATED, int MT, bool DIRECT = false>
__device__ __forceinline__ void grouped_dot_body(const uint16_t* __restrict__ a, int64_t lda,
                                                 const int32_t* __restrict__ sorted, int32_t top_k, const MoeTile& ent,
                                                 int32_t t, const uint8_t* __restrict__ wt, int32_t rows_per_expert,
                                                 int32_t K, const float* __restrict__ alpha_e,
                                                 const float* __restrict__ topk_w, void* __restrict__ out, int64_t ldo,
                                                 float* __restrict__ red) {
  constexpr int R = GATED ? 2 : 1;
  const int lane = int(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int q = lane >> 4, n = lane & 15;
  const int32_t steps = K / 256;
  const int32_t tiles_e = rows_per_expert / 16;
  const int32_t wtile[2] = {ent.expert * tiles_e + t, ent.expert * tiles_e + tiles_e / 2 + t};  // gate, up
  const int koff = 64 * (n >> 2) + 16 * q + 8 * ((n >> 1) & 1) + 4 * (n & 1);
  const uint16_t* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int32_t slot = ent.slot0 + m;
    // DIRECT: each pair is its own entry, its slot the pair index itself
    arow[m] = a + int64_t(GATED ? (DIRECT ? slot : sorted[slot]) / top_k : slot) * lda + koff;
  }
  auto unit_at = [&](int r, int32_t st) {
    return load_unit(wt + (int64_t(wtile[r]) * steps + min(st, steps - 1)) * kUnitBytes, lane);
  };
  auto act_at = [&](int32_t st, uint2 (&x)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) x[m] = *reinterpret_cast<const uint2*>(arow[m] + 256 * int64_t(min(st, steps - 1)));
  };
  float alpha = alpha_e[ent.expert];
  Unit w[2][R];
  uint2 x[2][MT];
  act_at(wave, x[0]);
#pragma unroll
  for (int r = 0; r < R; ++r) w[0][r] = unit_at(r, wave);
  if (PER > 1) {
    act_at(wave + nwaves, x[1]);
#pragma unroll
    for (int r = 0; r < R; ++r) w[1][r] = unit_at(r, wave + nwaves);
  }
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (wave + i * nwaves < steps) {
#pragma unroll
      for (int r = 0; r < R; ++r) dot_step<MT>(w[i & 1][r], x[i & 1], acc[r]);
    }
    if (i + 2 < PER) {
      act_at(wave + (i + 2) * nwaves, x[i & 1]);
#pragma unroll
      for (int r = 0; r < R; ++r) w[i & 1][r] = unit_at(r, wave + (i + 2) * nwaves);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the row's 4 lanes (q), then the waves in order
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[r][m] += __shfl_xor(acc[r][m], 16, 64);
      acc[r][m] += __shfl_xor(acc[r][m], 32, 64);
    }
  if (nwaves > 1) {
    if (q == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) red[((wave * R + r) * MT + m) * 16 + n] = acc[r][m];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        acc[r][m] = red[(r * MT + m) * 16 + n];
        for (int k = 1; k < nwaves; ++k) acc[r][m] += red[((k * R + r) * MT + m) * 16 + n];
      }
  }
  if (q != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int32_t slot = ent.slot0 + m;
    const int64_t at = int64_t(slot) * ldo + 16 * t + n;
    if (GATED) {
      const float h = silu(alpha * acc[0][m]) * (alpha * acc[R - 1][m]);
      static_cast<uint16_t*>(out)[at] = __builtin_bit_cast(uint16_t, (__bf16)h);
    } else {
      static_cast<float*>(out)[at] = topk_w[sorted[slot]] * (alpha * acc[0][m]);
    }
  }
}

template <int PER, bool GATED>
__global__ __launch_bounds__(512) void w4a16_grouped_kernel(
    const uint16_t* __restrict__ a, int64_t lda, const int32_t* __restrict__ sorted, int32_t top_k,
    const MoeTile* __restrict__ entries, int32_t out_tiles, const uint8_t* __restrict__ wt, int32_t rows_per_expert,
    int32_t K, const float* __restrict__ alpha_e, const float* __restrict__ topk_w, void* __restrict__ out,
    int64_t ldo) {
  constexpr int R = GATED ? 2 : 1;
  extern __shared__ float red[];  // [waves][R][64][4]
  const int32_t entry = int32_t(blockIdx.x) / out_tiles, t = int32_t(blockIdx.x) - entry * out_tiles;
  const MoeTile ent = entries[entry];
  if (ent.rows <= 0) return;
  if (ent.rows == 1) {
    grouped_dot_body<PER, GATED, 1>(a, lda, sorted, top_k, ent, t, wt, rows_per_expert, K, alpha_e, topk_w, out, ldo,
                                    red);
    return;
  }
  if (ent.rows == 2) {
    grouped_dot_body<PER, GATED, 2>(a, lda, sorted, top_k, ent, t, wt, rows_per_expert, K, alpha_e, topk_w, out, ldo,
                                    red);
    return;
  }
  const int lane = int(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int q = lane >> 4;
  const int32_t steps = K / 256;
  const int32_t tiles_e = rows_per_expert / 16;
  const int32_t wtile0 = ent.expert * tiles_e + t, wtile1 = wtile0 + tiles_e / 2;  // gate, up
  // permuted activation loads: lane 4c + q loads what MFMA lane c + 16q needs
  const int lrow = lane >> 2, lq = lane & 3;
  const int src_byte = 4 * (4 * (lane & 15) + q);
  int32_t arow = -1;
  if (lrow < ent.rows) arow = GATED ? sorted[ent.slot0 + lrow] / top_k : ent.slot0 + lrow;
  const __amdgpu_buffer_rsrc_t arsrc = act_rsrc(a);
  const uint32_t aoff = arow >= 0 ? uint32_t(arow) * uint32_t(lda) * 2u + 32u * uint32_t(lq) : 0x80000000u;
  auto unit_at = [&](int r, int32_t st) {
    return load_unit(wt + (int64_t(r == 0 ? wtile0 : wtile1) * steps + min(st, steps - 1)) * kUnitBytes, lane);
  };
  auto b_at = [&](int32_t st) { return load_b_rows(arsrc, aoff, min(st, steps - 1)); };

  f32x4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Unit w[2][R];
  StepB b[2];
  float alpha = alpha_e[ent.expert];
#pragma unroll
  for (int r = 0; r < R; ++r) w[0][r] = unit_at(r, wave);
  b[0] = b_at(wave);
  __builtin_amdgcn_sched_barrier(0);
  settle(alpha);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (i + 1 < PER) {
#pragma unroll
      for (int r = 0; r < R; ++r) w[(i + 1) & 1][r] = unit_at(r, wave + (i + 1) * nwaves);
      b[(i + 1) & 1] = b_at(wave + (i + 1) * nwaves);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool live = wave + i * nwaves < steps;
    const StepB& bs = b[i & 1];
    uint4 b0[4], b1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0[j] = to_mfma_lane(bs.v[j], src_byte);
      b1[j] = to_mfma_lane(bs.v[4 + j], src_byte);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      mma_half(w[i & 1][r].c0, w[i & 1][r].sc, 0, b0, acc[r], live);
      mma_half(w[i & 1][r].c1, w[i & 1][r].sc, 1, b1, acc[r], live);
    }
  }
  // partial tiles added through LDS in wave order
  if (nwaves > 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<f32x4_t*>(&red[((wave * R + r) * 64 + lane) * 4]) = acc[r];
    __syncthreads();
    if (wave != 0) return;
    for (int w2 = 1; w2 < nwaves; ++w2)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += *reinterpret_cast<const f32x4_t*>(&red[((w2 * R + r) * 64 + lane) * 4]);
  }
  // lane (c, qq) holds rows 16t + 4qq + i of token column c
  const int c = lane & 15, qq = lane >> 4;
  if (c >= ent.rows) return;
  const int32_t slot = ent.slot0 + c;
  const int64_t at = int64_t(slot) * ldo + 16 * t + 4 * qq;
  if (GATED) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = silu(alpha * acc[0][i]) * (alpha * acc[R - 1][i]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + at) =
        make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
  } else {
    const float wr = topk_w[sorted[slot]];
    *reinterpret_cast<float4*>(static_cast<float*>(out) + at) =
        make_float4(wr * (alpha * acc[0][0]), wr * (alpha * acc[0][1]), wr * (alpha * acc[0][2]),
                    wr * (alpha * acc[0][3]));
  }
}

// ------------------------------------------------------- direct (decode)
// The W4A16 MoE layer when every pair can be its own entry (few pairs): no
// align.  gate_up: one workgroup per (pair, 16-row gate tile) on the dot
// products of a one-pair entry, reading the pair's expert from the routing
// ids and storing h at the pair index.  Skipped pairs (ids outside [0, E))
// store nothing.
template <int PER>
__global__ __launch_bounds__(512) void w4a16_direct_gate_up_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ ids, int32_t top_k, int32_t E,
    int32_t out_tiles, const uint8_t* __restrict__ wt, int32_t rows_per_expert, int32_t K,
    const float* __restrict__ alpha_e, uint16_t* __restrict__ h, int64_t ldh) {
  extern __shared__ float red[];  // [waves][2][1][16]
  const int32_t p = int32_t(blockIdx.x) / out_tiles, t = int32_t(blockIdx.x) - p * out_tiles;
  const int32_t e = ids[p];
  if (e < 0 || e >= E) return;
  MoeTile ent;
  ent.expert = e;
  ent.slot0 = p;
  ent.rows = 1;
  ent.pad = 0;
  grouped_dot_body<PER, true, 1, true>(x, ldx, nullptr, top_k, ent, t, wt, rows_per_expert, K, alpha_e, nullptr, h,
                                       ldh, red);
}

// down and the route sum in one launch: workgroup (token t, 16-row output
// tile) has one wave per route r.  Wave r computes y_r = w[t, r] *
// (alpha_dn[e] * (h[t*top_k + r] . W_dn[e] rows)) over I with the dot
// products of the dot schedule (PER = I/256 steps, two in flight); wave 0 then
// adds the token's routes in the order r = 0, 1, ... in fp32 (skipped routes
// add nothing) and rounds once to bf16 -- the route sum of the grouped path.
template <int PER>
__global__ __launch_bounds__(1024) void w4a16_direct_down_sum_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
    int32_t top_k, int32_t E, const uint8_t* __restrict__ wt, int32_t K, int32_t I,
    const float* __restrict__ alpha_e, uint16_t* __restrict__ out, int64_t ldo) {
  __shared__ float ys[16][16];  // [route][output row of the tile]
  __shared__ int32_t live_r[16];
  const int lane = int(threadIdx.x & 63);
  const int r = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int q = lane >> 4, n = lane & 15;
  const int32_t tiles_e = K / 16;  // output tiles of one expert's down bank
  const int32_t t = int32_t(blockIdx.x) / tiles_e, tile = int32_t(blockIdx.x) - t * tiles_e;
  const int32_t p = t * top_k + r;
  const int32_t e = ids[p];
  const bool live = e >= 0 && e < E;  // uniform per wave
  float y = 0.0f;
  if (live) {
    const uint8_t* wtile = wt + (int64_t(e) * tiles_e + tile) * PER * kUnitBytes;
    const int koff = 64 * (n >> 2) + 16 * q + 8 * ((n >> 1) & 1) + 4 * (n & 1);
    const uint16_t* arow = h + int64_t(p) * I + koff;
    const float alpha = alpha_e[e];
    Unit w[2];
    uint2 xa[2][1];
    w[0] = load_unit(wtile, lane);
    xa[0][0] = *reinterpret_cast<const uint2*>(arow);
    if (PER > 1) {
      w[1] = load_unit(wtile + kUnitBytes, lane);
      xa[1][0] = *reinterpret_cast<const uint2*>(arow + 256);
    }
    float acc[1] = {0.0f};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dot_step<1>(w[i & 1], xa[i & 1], acc);
      if (i + 2 < PER) {
        w[i & 1] = load_unit(wtile + (i + 2) * kUnitBytes, lane);
        xa[i & 1][0] = *reinterpret_cast<const uint2*>(arow + 256 * (i + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    acc[0] += __shfl_xor(acc[0], 16, 64);
    acc[0] += __shfl_xor(acc[0], 32, 64);
    y = topk_w[p] * (alpha * acc[0]);
  }
  if (lane == 0) live_r[r] = live ? 1 : 0;
  if (q == 0) ys[r][n] = y;
  __syncthreads();
  if (r != 0 || q != 0) return;
  float sum = 0.0f;
  for (int rr = 0; rr < top_k; ++rr)
    if (live_r[rr]) sum += ys[rr][n];
  out[int64_t(t) * ldo + 16 * tile + n] = __builtin_bit_cast(uint16_t, (__bf16)sum);
}

std::atomic<int> g_cu_count[64];

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

int cu_count() { return device_cu_count(); }

}  // namespace

namespace {

// Steps per wave and waves per workgroup for a requested ksplit (no wave is
// left without a step).
struct SplitShape {
  int64_t per, waves;
};
// LDS token rows of the shared schedule: M for one token group, else M
// padded to its 16-row token groups.
int64_t shared_rows(int64_t M) { return M <= 16 ? std::max<int64_t>(1, M) : 16 * ((M + 15) / 16); }

SplitShape split_shape(int64_t ksplit, int64_t steps) {
  const int64_t ks = std::min<int64_t>(ksplit, steps);
  const int64_t per = (steps + ks - 1) / ks;
  return {per, (steps + per - 1) / per};
}

}  // namespace

W4A16Config w4a16_default_config(int64_t M, int64_t N, int64_t K) {
  const int64_t steps = K / 256;
  const int64_t tiles = std::max<int64_t>(1, (N + 15) / 16);
  const int64_t cus = cu_count();
  W4A16Config c;
  c.ksplit = 0;
  c.chunk_steps = 0;
  if (M > 16) {
    // more than one token group: only the shared schedule (16 M-row MFMA
    // columns per group, the weight dequantized once for all groups)
    c.schedule = 2;
    c.chunk_steps = int(std::max<int64_t>(1, std::min<int64_t>(steps, 64 / shared_rows(M))));
    return c;
  }
  if (M <= 2 || (M == 3 && tiles * steps >= 20 * cus && tiles < int64_t(kSharedTiles) * cus * 3 / 2)) {
    // dot: waves per tile so the launch gives every CU about 8 waves (at
    // least 4 per workgroup), and at most 2 steps per wave while there are at
    // most 2 tiles per CU.  At one or two tokens this also beats the shared
    // schedule on many tiles (N = 62080: the time of a plain read of the
    // weight at M = 1)
    int64_t ks = std::max<int64_t>({(8 * cus + tiles - 1) / tiles, (steps + kSplitMaxPer - 1) / kSplitMaxPer, 4});
    if (tiles <= 2 * cus) ks = std::max<int64_t>(ks, (steps + 1) / 2);
    // long K (more than 32 steps): at most about 4 steps per wave (measured
    // cold at K = 11008 and 14336: 5-8 % faster than 6-7 steps)
    if (steps > 32) ks = std::max<int64_t>(ks, (steps + 3) / 4);
    W4A16Config dot = c;
    dot.schedule = 4;
    dot.ksplit = int(std::min<int64_t>({ks, steps, 16}));
    // at most kSplitMaxPer steps per wave over at most 16 waves: above
    // K = 16 * 8 * 256 the split schedules below take the call
    if (w4a16_config_valid(dot, M, K)) return dot;
  }
  if (tiles >= int64_t(kSharedTiles) * cus * 3 / 2) {
    // shared: the largest chunk whose double buffer fits in 64 KiB of LDS
    c.schedule = 2;
    c.chunk_steps = int(std::max<int64_t>(1, std::min<int64_t>(steps, 64 / shared_rows(M))));
    // up to 8 tokens: two tiles per workgroup on 4 waves instead (measured
    // cold at N = 62080, K = 5120: M = 4 37.1 -> 34.8 us, M = 8 37.3 -> 37.0)
    W4A16Config two = c;
    two.schedule = 3;
    two.ksplit = 4;
    two.chunk_steps = 2;
    if (M <= 8 && w4a16_config_valid(two, M, K)) c = two;
  } else {
    // split: waves per tile so the launch gives every CU about 8 waves;
    // interleaved steps while a wave has at most kSplitMaxPer of them.  With
    // between one and two tiles per CU, two tiles per workgroup on 4 waves
    // (each step's activation operands serve both; measured 4-20 % faster at
    // 320 tiles, slower at 224 and within noise at 544)
    int64_t want = (8 * cus + tiles - 1) / tiles;
    if (steps > 32) want = std::max<int64_t>(want, (steps + 3) / 4);  // long K: about 4 steps per wave
    c.ksplit = int(std::max<int64_t>(1, std::min<int64_t>({want, steps, 16})));
    const int64_t ks = std::min<int64_t>(c.ksplit, steps);
    c.schedule = (steps + ks - 1) / ks <= kSplitMaxPer ? 3 : 1;
    W4A16Config three = c;
    three.schedule = 3;
    three.chunk_steps = 3;
    three.ksplit = int(std::max<int64_t>(4, (steps + kSplitMaxPer - 1) / kSplitMaxPer));
    if (tiles > 2 * cus && tiles <= 3 * cus && w4a16_config_valid(three, M, K)) {
      // between 2 and 3 tiles per CU: one workgroup per CU holding 2 or 3
      // tiles, each step's activation operands serving all of them (measured
      // cold: 8704 x 5120 at M = 4/8/16 from 10.3/11.2/14.0 to 8.6/9.6/10.3
      // us; 11008 x 4096 7-14 % faster)
      c = three;
    } else if (c.schedule == 3 && tiles > cus && tiles <= 2 * cus) {
      W4A16Config two = c;
      two.chunk_steps = 2;
      two.ksplit = int(std::max<int64_t>(std::min<int64_t>(4, steps), (steps + kSplitMaxPer - 1) / kSplitMaxPer));
      if (w4a16_config_valid(two, M, K)) c = two;
    } else if (tiles > 2 * cus + cus / 2) {
      // more than 2.5 tiles per CU: two tiles per workgroup on 8 waves
      // (measured cold at N = 11008, 14336 and 28672, K = 4096: 15-37 %
      // faster than one tile per workgroup; neutral at 2.1 tiles per CU)
      W4A16Config two = c;
      two.schedule = 3;
      two.chunk_steps = 2;
      two.ksplit = int(std::min<int64_t>(8, steps));
      if (w4a16_config_valid(two, M, K)) c = two;
    }
  }
  return c;
}

bool w4a16_config_valid(const W4A16Config& c, int64_t M, int64_t K) {
  if (M > kW4A16MaxM || (M > 16 && c.schedule != 2)) return false;
  if (c.cache_policy < 0 || c.cache_policy > 2 || (c.cache_policy != 0 && c.schedule != 4)) return false;
  if (c.schedule == 1) return c.ksplit >= 1 && c.ksplit <= 16;
  if (c.schedule == 3) {
    // chunk_steps: tiles per workgroup (0 or 1: one; 2: two, at most 8 waves)
    const int64_t steps = K / 256;
    if (c.ksplit < 1 || c.ksplit > 16 || c.chunk_steps < 0 || c.chunk_steps > 3) return false;
    const SplitShape sh = split_shape(c.ksplit, steps);
    // two tiles: at most 8 waves; 2-3 tiles: 3 to 8 waves (wave r adds up tile r)
    return sh.per <= kSplitMaxPer && (c.chunk_steps < 2 || sh.waves <= 8) && (c.chunk_steps < 3 || sh.waves >= 3);
  }
  if (c.schedule == 4) {
    if (M > kDotMaxM || c.ksplit < 1 || c.ksplit > 16) return false;
    return split_shape(c.ksplit, K / 256).per <= kSplitMaxPer;
  }
  if (c.schedule == 2) {
    if (c.chunk_steps < 1) return false;
    const int64_t kc = std::min<int64_t>(c.chunk_steps, K / 256);
    // 16-byte entries: LDS (rows padded to the token groups), staging registers (real rows)
    return 2 * shared_rows(M) * kc * 32 * 16 <= 64 * 1024 && std::max<int64_t>(1, M) * kc * 32 <= 4 * kSharedTiles * 64;
  }
  return false;
}

hipError_t launch_w4a16(const void* a, int64_t M, int64_t lda, const void* w_tiled, int64_t N, int64_t K,
                        const float* alpha, void* out, int64_t ldo, const W4A16Config& cfg, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t steps = K / 256;
  const int64_t tiles = (N + 15) / 16;
  const auto* A = static_cast<const uint16_t*>(a);
  const auto* WT = static_cast<const uint8_t*>(w_tiled);
  auto* O = static_cast<uint16_t*>(out);
  if (cfg.schedule == 2) {
    const int64_t kc = std::min<int64_t>(cfg.chunk_steps, steps);
    const size_t lds = 2 * size_t(shared_rows(M)) * size_t(kc) * 32 * 16;
    // 16 tiles per workgroup on weights of at least 1.5 x 8 tiles per CU
    // (measured cold at N = 62080, K = 5120: M = 16/32/64 46.2/64.6/100.1 ->
    // 41.9/57.1/80.7 us against 8 tiles); 8 below, where 16 would leave CUs idle
    const bool wide = tiles >= int64_t(kSharedTiles) * cu_count() * 3 / 2;
    const int tpw = wide ? 2 * kSharedTiles : kSharedTiles;
    const int64_t groups = (tiles + tpw - 1) / tpw;
    const dim3 grid{uint32_t(groups)}, block{uint32_t(64 * tpw)};
#define NVFP4_SHARED_LAUNCH(MG)                                                                                  \
  do {                                                                                                           \
    if (wide)                                                                                                    \
      hipLaunchKernelGGL((w4a16_shared_kernel<MG, 2 * kSharedTiles>), grid, block, lds, stream, A, lda,          \
                         int32_t(M), WT, int32_t(N), int32_t(K), int32_t(kc), alpha, O, ldo);                    \
    else                                                                                                         \
      hipLaunchKernelGGL((w4a16_shared_kernel<MG, kSharedTiles>), grid, block, lds, stream, A, lda, int32_t(M),  \
                         WT, int32_t(N), int32_t(K), int32_t(kc), alpha, O, ldo);                                \
  } while (0)
    if (M <= 16) NVFP4_SHARED_LAUNCH(1);
    else if (M <= 32) NVFP4_SHARED_LAUNCH(2);
    else if (M <= 48) NVFP4_SHARED_LAUNCH(3);
    else NVFP4_SHARED_LAUNCH(4);
#undef NVFP4_SHARED_LAUNCH
    return hipGetLastError();
  }
  if (cfg.schedule == 4) {
    const SplitShape sh = split_shape(cfg.ksplit, steps);
    const size_t lds = size_t(16) * kDotMaxM * 16 * sizeof(float);
    const dim3 grid{uint32_t(tiles)}, block{uint32_t(64 * sh.waves)};
#define NVFP4_DOT_LAUNCH(P, MT, CP)                                                                              \
  hipLaunchKernelGGL((w4a16_dot_kernel<P, MT, CP>), grid, block, lds, stream, A, lda, int32_t(M), WT, int32_t(N),\
                     int32_t(K), alpha, O, ldo)
#define NVFP4_DOT_M(P, CP)                                                                                       \
    if (M == 1) NVFP4_DOT_LAUNCH(P, 1, CP); else if (M == 2) NVFP4_DOT_LAUNCH(P, 2, CP);                         \
    else if (M == 3) NVFP4_DOT_LAUNCH(P, 3, CP); else NVFP4_DOT_LAUNCH(P, 4, CP);
#define NVFP4_DOT(P)                                                                                             \
  case P:                                                                                                        \
    if (cfg.cache_policy == 1) { NVFP4_DOT_M(P, 1) }                                                             \
    else if (cfg.cache_policy == 2) { NVFP4_DOT_M(P, 2) }                                                        \
    else { NVFP4_DOT_M(P, 0) }                                                                                   \
    return hipGetLastError();
    switch (sh.per) {
      NVFP4_DOT(1)
      NVFP4_DOT(2)
      NVFP4_DOT(3)
      NVFP4_DOT(4)
      NVFP4_DOT(5)
      NVFP4_DOT(6)
      NVFP4_DOT(7)
      NVFP4_DOT(8)
      default:
        return hipErrorInvalidValue;
    }
#undef NVFP4_DOT
#undef NVFP4_DOT_M
#undef NVFP4_DOT_LAUNCH
  }
  // contiguous runs of steps per wave; no wave is left without a step
  const int64_t ks = std::min<int64_t>(cfg.ksplit, steps);
  const int64_t per = (steps + ks - 1) / ks;
  const int waves = int((steps + per - 1) / per);
  // tiles per workgroup: 1, 2, or (chunk_steps 3) 2 to 3 on about one
  // workgroup per CU: G workgroups, the first `full` of them with 3 tiles
  const int R = cfg.schedule == 3 && cfg.chunk_steps >= 2 ? cfg.chunk_steps : 1;
  int64_t G = (tiles + R - 1) / R, full = G;
  if (R == 3) {
    G = std::max<int64_t>(std::min<int64_t>(cu_count(), tiles / 2), (tiles + 2) / 3);
    full = std::max<int64_t>(0, tiles - 2 * G);
  }
  const size_t lds = waves > 1 ? size_t(waves) * R * 64 * 4 * sizeof(float) : 0;
  const dim3 grid{uint32_t(G)}, block{uint32_t(64 * waves)};
  // permuted activation loads once several token rows share a load group
  const bool perm = M > 4;
#define NVFP4_SPLIT_LAUNCH(P, IL, PM, RR)                                                                       \
  hipLaunchKernelGGL((w4a16_split_fixed_kernel<P, IL, PM, RR>), grid, block, lds, stream, A, lda, int32_t(M),   \
                     WT, int32_t(N), int32_t(K), int32_t(per), alpha, O, ldo, int32_t(full))
#define NVFP4_SPLIT_FIXED(P)                                                                                    \
  case P:                                                                                                       \
    if (cfg.schedule == 3 && R == 3) {                                                                          \
      if (perm) NVFP4_SPLIT_LAUNCH(P, true, true, 3); else NVFP4_SPLIT_LAUNCH(P, true, false, 3);               \
    } else if (cfg.schedule == 3 && R == 2) {                                                                   \
      if (perm) NVFP4_SPLIT_LAUNCH(P, true, true, 2); else NVFP4_SPLIT_LAUNCH(P, true, false, 2);               \
    } else if (cfg.schedule == 3) {                                                                             \
      if (perm) NVFP4_SPLIT_LAUNCH(P, true, true, 1); else NVFP4_SPLIT_LAUNCH(P, true, false, 1);               \
    } else {                                                                                                    \
      if (perm) NVFP4_SPLIT_LAUNCH(P, false, true, 1); else NVFP4_SPLIT_LAUNCH(P, false, false, 1);             \
    }                                                                                                           \
    return hipGetLastError();
  switch (per) {
    NVFP4_SPLIT_FIXED(1)
    NVFP4_SPLIT_FIXED(2)
    NVFP4_SPLIT_FIXED(3)
    NVFP4_SPLIT_FIXED(4)
    NVFP4_SPLIT_FIXED(5)
    NVFP4_SPLIT_FIXED(6)
    NVFP4_SPLIT_FIXED(7)
    NVFP4_SPLIT_FIXED(8)
    default:
      break;
  }
#undef NVFP4_SPLIT_FIXED
#undef NVFP4_SPLIT_LAUNCH
  hipLaunchKernelGGL(w4a16_split_kernel, grid, block, lds, stream, A, lda, int32_t(M), WT, int32_t(N), int32_t(K),
                     int32_t(per), alpha, O, ldo);
  return hipGetLastError();
}

hipError_t launch_w4a16_grouped(bool gated, const void* a, int64_t lda, const int32_t* sorted, int64_t top_k,
                                const MoeTile* entries, int64_t n_entries, int64_t out_tiles, const void* w_tiled,
                                int64_t rows_per_expert, int64_t K, const float* alpha_e, const float* topk_w,
                                void* out, int64_t ldo, hipStream_t stream) {
  if (n_entries == 0 || out_tiles == 0) return hipSuccess;
  const int64_t steps = K / 256;
  const int64_t waves = std::min<int64_t>(steps, 8);
  const int64_t per = (steps + waves - 1) / waves;
  const size_t lds = waves > 1 ? size_t(waves) * (gated ? 2 : 1) * 64 * 4 * sizeof(float) : 0;
  const dim3 grid{uint32_t(n_entries * out_tiles)}, block{uint32_t(64 * waves)};
  const auto* A = static_cast<const uint16_t*>(a);
  const auto* WT = static_cast<const uint8_t*>(w_tiled);
#define NVFP4_GROUPED(P)                                                                                       \
  case P:                                                                                                      \
    if (gated)                                                                                                 \
      hipLaunchKernelGGL((w4a16_grouped_kernel<P, true>), grid, block, lds, stream, A, lda, sorted,            \
                         int32_t(top_k), entries, int32_t(out_tiles), WT, int32_t(rows_per_expert), int32_t(K), \
                         alpha_e, topk_w, out, ldo);                                                           \
    else                                                                                                       \
      hipLaunchKernelGGL((w4a16_grouped_kernel<P, false>), grid, block, lds, stream, A, lda, sorted,           \
                         int32_t(top_k), entries, int32_t(out_tiles), WT, int32_t(rows_per_expert), int32_t(K), \
                         alpha_e, topk_w, out, ldo);                                                           \
    return hipGetLastError();
  switch (per) {
    NVFP4_GROUPED(1)
    NVFP4_GROUPED(2)
    NVFP4_GROUPED(3)
    NVFP4_GROUPED(4)
    NVFP4_GROUPED(5)
    NVFP4_GROUPED(6)
    NVFP4_GROUPED(7)
    NVFP4_GROUPED(8)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_GROUPED
}

hipError_t launch_w4a16_moe_direct(const void* x, int64_t ldx, const int32_t* ids, int64_t T, int64_t top_k,
                                   int64_t E, int64_t I, const void* w_gate_up, const void* w_down, int64_t K,
                                   const float* alpha_gu, const float* alpha_dn, const float* topk_w, void* h,
                                   void* out, int64_t ldo, hipStream_t stream) {
  const int64_t P = T * top_k;
  if (P == 0) return hipSuccess;
  const auto* X = static_cast<const uint16_t*>(x);
  auto* H = static_cast<uint16_t*>(h);
  // gate_up: K/256 steps over up to 8 waves, as the grouped kernels
  {
    const int64_t steps = K / 256;
    const int64_t waves = std::min<int64_t>(steps, 8);
    const int64_t per = (steps + waves - 1) / waves;
    const size_t lds = size_t(waves) * 2 * 16 * sizeof(float);
    const dim3 grid{uint32_t(P * (I / 16))}, block{uint32_t(64 * waves)};
    const auto* WT = static_cast<const uint8_t*>(w_gate_up);
#define NVFP4_DIRECT_GU(PP)                                                                                    \
  case PP:                                                                                                     \
    hipLaunchKernelGGL((w4a16_direct_gate_up_kernel<PP>), grid, block, lds, stream, X, ldx, ids, int32_t(top_k), \
                       int32_t(E), int32_t(I / 16), WT, int32_t(2 * I), int32_t(K), alpha_gu, H, I);           \
    break;
    switch (per) {
      NVFP4_DIRECT_GU(1)
      NVFP4_DIRECT_GU(2)
      NVFP4_DIRECT_GU(3)
      NVFP4_DIRECT_GU(4)
      NVFP4_DIRECT_GU(5)
      NVFP4_DIRECT_GU(6)
      NVFP4_DIRECT_GU(7)
      NVFP4_DIRECT_GU(8)
      default:
        return hipErrorInvalidValue;
    }
#undef NVFP4_DIRECT_GU
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // down + route sum: one wave per route, I/256 steps each
  const dim3 grid{uint32_t(T * (K / 16))}, block{uint32_t(64 * top_k)};
  const auto* WD = static_cast<const uint8_t*>(w_down);
  auto* O = static_cast<uint16_t*>(out);
#define NVFP4_DIRECT_DN(PP)                                                                                    \
  case PP:                                                                                                     \
    hipLaunchKernelGGL((w4a16_direct_down_sum_kernel<PP>), grid, block, 0, stream, H, ids, topk_w,             \
                       int32_t(top_k), int32_t(E), WD, int32_t(K), int32_t(I), alpha_dn, O, ldo);              \
    break;
  switch (I / 256) {
    NVFP4_DIRECT_DN(1)
    NVFP4_DIRECT_DN(2)
    NVFP4_DIRECT_DN(3)
    NVFP4_DIRECT_DN(4)
    NVFP4_DIRECT_DN(5)
    NVFP4_DIRECT_DN(6)
    NVFP4_DIRECT_DN(7)
    NVFP4_DIRECT_DN(8)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_DIRECT_DN
  return hipGetLastError();
}

}  // namespace nvfp4
