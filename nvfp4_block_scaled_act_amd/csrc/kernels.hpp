// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

hipError_t launch_quantize(const void* a, int64_t M, int64_t K, int64_t lda, const float* g, void* codes,
                           void* scales, hipStream_t stream);
hipError_t launch_global_scale(const void* x, int64_t rows, int64_t cols, int64_t ld, float* g_out,
                               hipStream_t stream);
hipError_t launch_alpha(const float* g_w, const float* g_a, float* alpha, hipStream_t stream);

// Re-tiling of a canonical [N, K/2] + [N, K/16] weight into the tiled layout
// both linears read (K % 256 == 0); tiled_weight_bytes is its size.
int64_t tiled_weight_bytes(int64_t N, int64_t K);
hipError_t launch_retile(const void* codes, const void* scales, int64_t N, int64_t K, void* dst, hipStream_t stream);

// W4A16 skinny kernel: out[M, N] = bf16(alpha * a[M, K] @ dequant(W)^T), M <= 16.
struct W4A16Config {
  int schedule;     // 1 = split (one tile per workgroup, K split over its waves), 2 = shared (8 tiles, all of K)
  int ksplit;       // split: waves per tile, 1..16
  int chunk_steps;  // shared: 256-k steps per LDS activation chunk
};
W4A16Config w4a16_default_config(int64_t M, int64_t N, int64_t K);
bool w4a16_config_valid(const W4A16Config& c, int64_t M, int64_t K);
hipError_t launch_w4a16(const void* a, int64_t M, int64_t lda, const void* w_tiled, int64_t N, int64_t K,
                        const float* alpha, void* out, int64_t ldo, const W4A16Config& cfg, hipStream_t stream);

// W4A4 tiled GEMM: out[M, N] = bf16(alpha * dequant(A)[M, K] @ dequant(W)^T).
hipError_t launch_w4a4(const void* a_codes, const void* a_scales, int64_t M, const void* w_tiled, int64_t N,
                       int64_t K, const float* alpha, void* out, int64_t ldo, hipStream_t stream);

}  // namespace nvfp4
