// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// swz_cols > 0: scales in the 128x4-swizzled layout with swz_cols (K/16
// rounded up to 4) scale columns, padding rows and columns written as zero.
hipError_t launch_quantize(const void* a, int64_t M, int64_t K, int64_t lda, const float* g, void* codes,
                           void* scales, hipStream_t stream, int64_t swz_cols = 0);
hipError_t launch_global_scale(const void* x, int64_t rows, int64_t cols, int64_t ld, float* g_out,
                               hipStream_t stream);
hipError_t launch_alpha(const float* g_w, const float* g_a, float* alpha, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// Re-tiling of a canonical [N, K/2] + [N, K/16] weight into the tiled layout
// both linears read (K % 256 == 0); tiled_weight_bytes is its size.
int64_t tiled_weight_bytes(int64_t N, int64_t K);
hipError_t launch_retile(const void* codes, const void* scales, int64_t N, int64_t K, void* dst, hipStream_t stream,
                         int64_t swz_cols = 0);
// Byte offset of scale (row, col) in the 128x4-swizzled layout with cols_pad
// (a multiple of 4) scale columns: 512-byte blocks of 128 rows x 4 columns,
// row-major over the blocks; inside a block, row r and column c at
// 16 (r % 32) + 4 ((r / 32) % 4) + c % 4.
__host__ __device__ inline int64_t swizzled_scale_offset(int64_t row, int64_t col, int64_t cols_pad) {
  return ((row >> 7) * (cols_pad >> 2) + (col >> 2)) * 512 + (row & 31) * 16 + ((row >> 5) & 3) * 4 + (col & 3);
}

// W4A16 skinny kernel: out[M, N] = bf16(alpha * a[M, K] @ dequant(W)^T), M <=
// kW4A16MaxM (schedules 1, 3 and 4 take M <= 16; schedule 2 up to 64).
constexpr int64_t kW4A16MaxM = 64;
struct W4A16Config {
  int schedule;     // 1 = split (one tile per workgroup, K split over its waves), 2 = shared (8 tiles, all of K),
                    // 3 = split with interleaved steps, 4 = dot (split on the VALU, M <= 4)
  int ksplit;       // split, dot: waves per tile, 1..16
  int chunk_steps;  // shared: 256-k steps per LDS activation chunk
  int cache_policy = 0;  // dot only: 0 weights nontemporal, activations default (the default);
                         // 1 weights default; 2 activations nontemporal too
};
W4A16Config w4a16_default_config(int64_t M, int64_t N, int64_t K);
bool w4a16_config_valid(const W4A16Config& c, int64_t M, int64_t K);
hipError_t launch_w4a16(const void* a, int64_t M, int64_t lda, const void* w_tiled, int64_t N, int64_t K,
                        const float* alpha, void* out, int64_t ldo, const W4A16Config& cfg, hipStream_t stream);

// W4A4 tiled GEMM: out[M, N] = bf16(alpha * dequant(A)[M, K] @ dequant(W)^T).
// With partials (fp32, w4a4_partials_bytes(M, N, K) long) and
// w4a4_splits(M, N, K) > 1, K is split across workgroups into that many
// ranges of whole 256-k units whose fp32 partial tiles a second launch adds
// in range order; without, one launch over all of K.
hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, float* partials, hipStream_t stream);
int w4a4_splits(int64_t M, int64_t N, int64_t K);
size_t w4a4_partials_bytes(int64_t M, int64_t N, int64_t K);

// Bytes of the dispatched linear's quantized activations (codes, then scales,
// each part 256-byte aligned); its split-K partials follow them.
inline size_t linear_act_bytes(int64_t M, int64_t K) {
  const size_t codes = (size_t(M) * size_t(K / 2) + 255) / 256 * 256;
  const size_t scales = (size_t(M) * size_t(K / 16) + 255) / 256 * 256;
  return codes + scales;
}

// The allocation-free linear's scratch size (NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES,
// checked in api.cpp): the split decision keeps activations + partials within it,
// so that every entry point takes the same decision for a shape.
constexpr size_t kLinearScratchBytes = size_t(64) << 20;
constexpr size_t kSplitKMaxBytes = size_t(48) << 20;  // fp32 partials of one split-K call, at most

// Library-owned scratch of the allocation-free dispatched linear: its size,
// and the device address of the current device's copy (looked up once per
// device with hipGetSymbolAddress).
size_t scratch_capacity();
hipError_t scratch_pointer(void** out);

// Streaming-read diagnostic: reads `bytes` (a multiple of 16) once.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

// NVFP4 MoE expert layer (W4A4 gate_up with SiLU gate and NVFP4 re-quantization,
// W4A4 down with routing weights, fp32 route sum in a fixed order).  The workspace holds,
// at the offsets moe_layout gives (256-byte aligned parts):
struct MoeTile {
  int32_t expert, slot0, rows, pad;  // rows == 0: unused entry
};
struct MoeLayout {
  int64_t chunks;     // align chunks of 1024 pairs
  int64_t max_tiles;  // tile table length: T*top_k/256 + E
  int64_t x_codes, x_scales;  // quantized hidden states [T, K/2], [T, K/16]
  int64_t counts;     // int32 [chunks, E]: per-chunk counts, then scatter bases
  int64_t offsets;    // int32 [E + 1]: first slot of each expert's pairs, [E] = pairs kept
  int64_t tiles;      // MoeTile [max_tiles]
  int64_t sorted;     // int32 [T*top_k]: pair index t*top_k + r at each slot
  int64_t h_codes, h_scales;  // NVFP4 h by slot [T*top_k, I/2], [T*top_k, I/16]
  int64_t inv;        // int32 [T*top_k]: slot of each pair, -1 if skipped
  int64_t ys;         // fp32 [T*top_k, K]: routing-weighted down outputs by slot
  int64_t total;      // bytes
};
MoeLayout moe_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I);
hipError_t launch_moe_w4a4(const void* x, int64_t T, int64_t ldx, const int32_t* ids, const float* topk_w,
                           int64_t top_k, int64_t E, int64_t I, const void* w_gate_up, const void* w_down, int64_t K,
                           const float* g1, const float* g2, const float* alpha_gu, const float* alpha_dn, void* out,
                           int64_t ldo, void* ws, float* h_amax, hipStream_t stream);

// The same layer with W4A16 on both GEMMs (bf16 x, bf16 h), for decode-sized
// batches: entries of up to kW4A16Rows pairs of one expert.
constexpr int kW4A16Rows = 16;
struct MoeW4A16Layout {
  int64_t chunks, max_tiles;  // align chunks; tile table length T*top_k/16 + E
  int64_t counts, offsets, tiles, sorted, inv;  // as MoeLayout
  int64_t h;      // bf16 [T*top_k, I] by slot
  int64_t ys;     // fp32 [T*top_k, K]: routing-weighted down outputs by slot
  int64_t total;  // bytes
};
MoeW4A16Layout moe_w4a16_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I);
hipError_t launch_moe_w4a16(const void* x, int64_t T, int64_t ldx, const int32_t* ids, const float* topk_w,
                            int64_t top_k, int64_t E, int64_t I, const void* w_gate_up, const void* w_down,
                            int64_t K, const float* alpha_gu, const float* alpha_dn, void* out, int64_t ldo, void* ws,
                            hipStream_t stream);
// Grouped W4A16 over the entries of a tile table (gated: gate_up with SiLU
// gate into bf16 h; else down into routing-weighted fp32 y), one workgroup
// per (entry, 16-row output tile).
hipError_t launch_w4a16_grouped(bool gated, const void* a, int64_t lda, const int32_t* sorted, int64_t top_k,
                                const MoeTile* entries, int64_t n_entries, int64_t out_tiles, const void* w_tiled,
                                int64_t rows_per_expert, int64_t K, const float* alpha_e, const float* topk_w,
                                void* out, int64_t ldo, hipStream_t stream);

// The W4A16 MoE layer for at most kMoeDirectPairs pairs (top_k <= 16, I and
// K/256 steps <= 8 x 8 and 8): gate_up per pair into bf16 h at the pair
// index (no align), then down and the fixed-order route sum in one launch.
constexpr int64_t kMoeDirectPairs = 64;  // NVFP4_MOE_W4A16_DIRECT_PAIRS (checked in api.cpp)
hipError_t launch_w4a16_moe_direct(const void* x, int64_t ldx, const int32_t* ids, int64_t T, int64_t top_k,
                                   int64_t E, int64_t I, const void* w_gate_up, const void* w_down, int64_t K,
                                   const float* alpha_gu, const float* alpha_dn, const float* topk_w, void* h,
                                   void* out, int64_t ldo, hipStream_t stream);

// Gated MLP gate_up on a dense NVFP4 batch: h = SiLU(z[:I]) * z[I:], z =
// alpha * deq(A) . deq(W_gu)^T, quantized to NVFP4 under g2 ([M, I/2] codes,
// [M, I/16] scales); h_amax (optional) receives max |h|.
hipError_t launch_gated_mlp_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_gate_up,
                                 int64_t K, int64_t I, const float* alpha, const float* g2, void* h_codes,
                                 void* h_scales, float* h_amax, hipStream_t stream);

}  // namespace nvfp4
