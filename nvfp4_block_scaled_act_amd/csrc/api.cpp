// C ABI of the NVFP4 library: host-side validation, the M-threshold dispatch
// and the calls into the gfx950 kernels.  Every check runs before any launch.
#include "../../include/nvfp4.h"

#include <algorithm>
#include <cmath>
#include <atomic>

#include "kernels.hpp"

static_assert(nvfp4::kMoeDirectPairs == NVFP4_MOE_W4A16_DIRECT_PAIRS, "direct-path threshold out of sync");
static_assert(nvfp4::kLinearScratchBytes == NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES, "scratch size out of sync");

namespace {

constexpr int64_t kInt32Max = 2147483647LL;
constexpr int64_t kW4a4MaxK = int64_t(1) << 24;  // the W4A4 kernels' 32-bit weight offsets
std::atomic<int64_t> g_route_m_max{16};  // measured crossover, N = 62080, K = 5120 (and most weights)
std::atomic<int64_t> g_moe_route_tpe_max{14};  // tokens per expert up to which the MoE stays W4A16

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Shape checks shared by prepare and the linears.
nvfp4_status check_weight_shape(int64_t N, int64_t K) {
  if (N < 0 || K <= 0) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 16 != 0) return NVFP4_ERR_INVALID_SHAPE;
  if (N > kInt32Max - 15 || K > kInt32Max) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 256 != 0) return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

// Checks shared by the linears: the prepared weight descriptor.
nvfp4_status check_weight(const nvfp4_weight* w) {
  if (!w) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight_shape(w->N, w->K);
  if (st != NVFP4_OK) return st;
  if (w->layout != NVFP4_LAYOUT_TILED) return NVFP4_ERR_UNSUPPORTED;
  if (w->N == 0) return NVFP4_OK;  // empty weight: data may be null
  if (!w->data) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!aligned16(w->data)) return NVFP4_ERR_ALIGNMENT;
  return NVFP4_OK;
}

nvfp4_status check_out(const void* out, int64_t M, int64_t N, int64_t ldo) {
  if (!out) return NVFP4_ERR_INVALID_ARGUMENT;
  if (ldo < N || ldo < 1) return NVFP4_ERR_INVALID_SHAPE;
  if (M > kInt32Max || (M > 0 && ldo > (INT64_MAX / 2) / M)) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned2(out)) return NVFP4_ERR_ALIGNMENT;
  return NVFP4_OK;
}

nvfp4_status check_bf16_input(const void* a, int64_t M, int64_t K, int64_t lda) {
  if (!a) return NVFP4_ERR_INVALID_ARGUMENT;
  if (lda < K) return NVFP4_ERR_INVALID_SHAPE;
  if (M > kInt32Max || K > kInt32Max) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(a) || lda % 8 != 0) return NVFP4_ERR_ALIGNMENT;
  return NVFP4_OK;
}

nvfp4_status w4a16_checked(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* alpha,
                           void* out, int64_t ldo, const nvfp4::W4A16Config* cfg_in, hipStream_t stream) {
  if (M < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  if (!alpha) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(w);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;  // empty batch: a and out may be null
  if ((st = check_bf16_input(a, M, w->K, lda)) != NVFP4_OK) return st;
  if ((st = check_out(out, M, w->N, ldo)) != NVFP4_OK) return st;
  if (M > nvfp4::kW4A16MaxM) return NVFP4_ERR_UNSUPPORTED;
  if ((M - 1) * lda * 2 + 2 * w->K > (int64_t(1) << 31) - 4096) return NVFP4_ERR_UNSUPPORTED;  // 32-bit offsets
  if (cfg_in && !nvfp4::w4a16_config_valid(*cfg_in, M, w->K)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (w->N == 0) return NVFP4_OK;
  const nvfp4::W4A16Config cfg = cfg_in ? *cfg_in : nvfp4::w4a16_default_config(M, w->N, w->K);
  if (!nvfp4::w4a16_config_valid(cfg, M, w->K)) return NVFP4_ERR_UNSUPPORTED;  // no schedule fits the shape
  return hip_status(nvfp4::launch_w4a16(a, M, lda, w->data, w->N, w->K, alpha, out, ldo, cfg, stream));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

const char* nvfp4_status_str(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4_ERR_INVALID_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported by this build's kernels";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int nvfp4_version(void) { return 100; }

#ifndef NVFP4_SOURCE_HASH
#define NVFP4_SOURCE_HASH "unknown"
#endif
const char* nvfp4_build_source_hash(void) { return NVFP4_SOURCE_HASH; }

nvfp4_status nvfp4_quantize_act(const void* a, int64_t M, int64_t K, int64_t lda, const float* g, void* codes,
                                void* scales, hipStream_t stream) {
  if (M < 0 || K <= 0) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 16 != 0 || lda < K) return NVFP4_ERR_INVALID_SHAPE;
  if (M == 0) return NVFP4_OK;  // empty batch: buffers may be null
  if (!g || !codes || !scales) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_bf16_input(a, M, K, lda);
  if (st != NVFP4_OK) return st;
  if (!aligned16(codes)) return NVFP4_ERR_ALIGNMENT;
  if (M * (K / 16) > kInt32Max) return NVFP4_ERR_INVALID_SHAPE;
  if ((M + 3) / 4 > 65535) return NVFP4_ERR_UNSUPPORTED;  // row mapping (grid.y), with margin
  if (M == 0) return NVFP4_OK;
  return hip_status(nvfp4::launch_quantize(a, M, K, lda, g, codes, scales, stream));
}

nvfp4_status nvfp4_global_scale(const void* x, int64_t rows, int64_t cols, int64_t ld, float* g_out,
                                hipStream_t stream) {
  if (!x || !g_out) return NVFP4_ERR_INVALID_ARGUMENT;
  if (rows < 0 || cols <= 0 || ld < cols) return NVFP4_ERR_INVALID_SHAPE;
  if (cols % 8 != 0 || ld % 8 != 0 || !aligned16(x) || (reinterpret_cast<uintptr_t>(g_out) & 3u))
    return NVFP4_ERR_ALIGNMENT;
  return hip_status(nvfp4::launch_global_scale(x, rows, cols, ld, g_out, stream));
}

nvfp4_status nvfp4_alpha(const float* g_w, const float* g_a, float* alpha_out, hipStream_t stream) {
  if (!g_w || !alpha_out) return NVFP4_ERR_INVALID_ARGUMENT;
  return hip_status(nvfp4::launch_alpha(g_w, g_a, alpha_out, stream));
}

nvfp4_status nvfp4_fused_weight_global(const float* g_parts, int64_t n_parts, float* g_out, int32_t* warn) {
  if (!g_parts || !g_out || n_parts <= 0) return NVFP4_ERR_INVALID_ARGUMENT;
  float lo = g_parts[0], hi = g_parts[0];
  for (int64_t i = 0; i < n_parts; ++i) {
    const float g = g_parts[i];
    if (!(g > 0.0f) || !std::isfinite(g)) return NVFP4_ERR_INVALID_ARGUMENT;
    lo = std::min(lo, g);
    hi = std::max(hi, g);
  }
  *g_out = hi;
  if (warn) *warn = double(hi) > 1.05 * double(lo) ? 1 : 0;
  return NVFP4_OK;
}

size_t nvfp4_swizzled_scales_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || K <= 0 || K % 16 != 0) return 0;
  return size_t((rows + 127) / 128 * 128) * size_t((K / 16 + 3) / 4 * 4);
}

nvfp4_status nvfp4_quantize_act_swizzled(const void* a, int64_t M, int64_t K, int64_t lda, const float* g,
                                         void* codes, void* scales, size_t scales_bytes, hipStream_t stream) {
  if (M < 0 || K <= 0) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 16 != 0 || lda < K) return NVFP4_ERR_INVALID_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!g || !codes || !scales) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_bf16_input(a, M, K, lda);
  if (st != NVFP4_OK) return st;
  if (!aligned16(codes)) return NVFP4_ERR_ALIGNMENT;
  const size_t need = nvfp4_swizzled_scales_bytes(M, K);
  if (scales_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (need > size_t(kInt32Max)) return NVFP4_ERR_INVALID_SHAPE;
  if ((M + 127) / 128 * 128 / 4 > 65535) return NVFP4_ERR_UNSUPPORTED;  // row mapping (grid.y)
  return hip_status(nvfp4::launch_quantize(a, M, K, lda, g, codes, scales, stream, (K / 16 + 3) / 4 * 4));
}

size_t nvfp4_prepared_weight_bytes(int64_t N, int64_t K) {
  if (check_weight_shape(N, K) != NVFP4_OK) return 0;
  return size_t(nvfp4::tiled_weight_bytes(N, K));
}

nvfp4_status nvfp4_prepare_weight(const void* codes, const void* scales, int64_t N, int64_t K, void* dst,
                                  size_t dst_bytes, nvfp4_weight* out, hipStream_t stream) {
  if (!out) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight_shape(N, K);
  if (st != NVFP4_OK) return st;
  const size_t need = size_t(nvfp4::tiled_weight_bytes(N, K));
  if (need > 0 && (!codes || !scales || !dst)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (dst_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && (!aligned16(dst) || (reinterpret_cast<uintptr_t>(codes) & 7u))) return NVFP4_ERR_ALIGNMENT;
  if (need > 0) {
    st = hip_status(nvfp4::launch_retile(codes, scales, N, K, dst, stream));
    if (st != NVFP4_OK) return st;
  }
  nvfp4_weight w;
  w.data = dst;
  w.N = N;
  w.K = K;
  w.layout = NVFP4_LAYOUT_TILED;
  w.reserved = 0;
  *out = w;
  return NVFP4_OK;
}

nvfp4_status nvfp4_prepare_weight_swizzled(const void* codes, const void* scales, size_t scales_bytes, int64_t N,
                                           int64_t K, void* dst, size_t dst_bytes, nvfp4_weight* out,
                                           hipStream_t stream) {
  if (!out) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight_shape(N, K);
  if (st != NVFP4_OK) return st;
  const size_t need = size_t(nvfp4::tiled_weight_bytes(N, K));
  if (need > 0 && (!codes || !scales || !dst)) return NVFP4_ERR_INVALID_ARGUMENT;
  if (dst_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && scales_bytes < nvfp4_swizzled_scales_bytes(N, K)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && (!aligned16(dst) || (reinterpret_cast<uintptr_t>(codes) & 7u))) return NVFP4_ERR_ALIGNMENT;
  if (need > 0) {
    st = hip_status(nvfp4::launch_retile(codes, scales, N, K, dst, stream, (K / 16 + 3) / 4 * 4));
    if (st != NVFP4_OK) return st;
  }
  nvfp4_weight w;
  w.data = dst;
  w.N = N;
  w.K = K;
  w.layout = NVFP4_LAYOUT_TILED;
  w.reserved = 0;
  *out = w;
  return NVFP4_OK;
}

nvfp4_status nvfp4_linear_w4a16(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* alpha,
                                void* out, int64_t ldo, hipStream_t stream) {
  return w4a16_checked(a, M, lda, w, alpha, out, ldo, nullptr, stream);
}

nvfp4_status nvfp4_linear_w4a16_ex(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w,
                                   const float* alpha, void* out, int64_t ldo, int schedule, int ksplit,
                                   int chunk_steps, int cache_policy, hipStream_t stream) {
  if (schedule == 0 && cache_policy == 0) return w4a16_checked(a, M, lda, w, alpha, out, ldo, nullptr, stream);
  if (schedule == 0) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4::W4A16Config cfg;
  cfg.schedule = schedule;
  cfg.ksplit = ksplit;
  cfg.chunk_steps = chunk_steps;
  cfg.cache_policy = cache_policy;
  return w4a16_checked(a, M, lda, w, alpha, out, ldo, &cfg, stream);
}

namespace {

// partials: fp32 room for the split-K ranges (nvfp4::w4a4_partials_bytes), or
// null for one launch over all of K.
nvfp4_status w4a4_checked(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* w,
                          const float* alpha, void* out, int64_t ldo, float* partials, hipStream_t stream) {
  if (M < 0 || !alpha) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(w);
  if (st != NVFP4_OK) return st;
  if (M == 0) return NVFP4_OK;  // empty batch: buffers may be null
  if (!a_codes || !a_scales) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((st = check_out(out, M, w->N, ldo)) != NVFP4_OK) return st;
  if (M > kInt32Max || M * (w->K / 16) > INT64_MAX / 16) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(a_codes) || !aligned16(a_scales)) return NVFP4_ERR_ALIGNMENT;
  // grid rows of 256 activation rows; 32-bit byte offsets into the codes
  if ((M + 255) / 256 > 65535 || M * (w->K / 2) >= (int64_t(1) << 32)) return NVFP4_ERR_UNSUPPORTED;
  // 32-bit byte offsets within a workgroup's 16 weight tiles (17 K/256 units)
  if (w->K > kW4a4MaxK) return NVFP4_ERR_UNSUPPORTED;
  if (w->N == 0) return NVFP4_OK;
  return hip_status(
      nvfp4::launch_w4a4(a_codes, a_scales, M, w->data, w->N, w->K, alpha, out, ldo, partials, stream));
}

}  // namespace

nvfp4_status nvfp4_linear_w4a4(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* w,
                               const float* alpha, void* out, int64_t ldo, hipStream_t stream) {
  return w4a4_checked(a_codes, a_scales, M, w, alpha, out, ldo, nullptr, stream);
}

size_t nvfp4_linear_w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return nvfp4::w4a4_partials_bytes(M, N, K);
}

nvfp4_status nvfp4_linear_w4a4_ws(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* w,
                                  const float* alpha, void* out, int64_t ldo, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  nvfp4_status st = check_weight(w);
  if (st != NVFP4_OK) return st;
  const size_t need = M > 0 ? nvfp4_linear_w4a4_workspace_bytes(M, w->N, w->K) : 0;
  if (need > 0) {
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(ws)) return NVFP4_ERR_ALIGNMENT;
  }
  return w4a4_checked(a_codes, a_scales, M, w, alpha, out, ldo, need > 0 ? static_cast<float*>(ws) : nullptr,
                      stream);
}

int nvfp4_route(int64_t M, int64_t N, int64_t K, int has_act_global) {
  (void)N;
  (void)K;
  return (has_act_global && M > g_route_m_max.load()) ? NVFP4_ROUTE_W4A4 : NVFP4_ROUTE_W4A16;
}

void nvfp4_set_route_m_max(int64_t m_max) {
  if (m_max < 0) m_max = 0;
  if (m_max > nvfp4::kW4A16MaxM) m_max = nvfp4::kW4A16MaxM;
  g_route_m_max.store(m_max);
}

int64_t nvfp4_get_route_m_max(void) { return g_route_m_max.load(); }

size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return nvfp4::linear_act_bytes(M, K) + (N > 0 ? nvfp4::w4a4_partials_bytes(M, N, K) : 0);
}

namespace {

// The dispatched linear; on the W4A4 route the quantized activations go to
// ws (ws_bytes long) -- the caller's workspace or the library's scratch.
nvfp4_status linear_impl(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* g_act,
                         const float* alpha_w4a16, const float* alpha_w4a4, void* out, int64_t ldo, void* ws,
                         size_t ws_bytes, bool use_scratch, int* route_taken, hipStream_t stream) {
  if (M < 0) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(w);
  if (st != NVFP4_OK) return st;
  const int route = nvfp4_route(M, w->N, w->K, g_act != nullptr);
  if (M == 0) {
    if (route_taken) *route_taken = route;
    return NVFP4_OK;
  }
  if (route == NVFP4_ROUTE_W4A16) {
    if (M > nvfp4::kW4A16MaxM) return NVFP4_ERR_UNSUPPORTED;
    st = w4a16_checked(a, M, lda, w, alpha_w4a16, out, ldo, nullptr, stream);
  } else {
    if (!alpha_w4a4) return NVFP4_ERR_INVALID_ARGUMENT;
    if ((st = check_bf16_input(a, M, w->K, lda)) != NVFP4_OK) return st;
    if ((st = check_out(out, M, w->N, ldo)) != NVFP4_OK) return st;
    const size_t need_act = nvfp4::linear_act_bytes(M, w->K);
    const size_t need = nvfp4_linear_workspace_bytes(M, w->N, w->K);
    if (M * (w->K / 16) > kInt32Max || (M + 3) / 4 > 65535 || (M + 255) / 256 > 65535 ||
        M * (w->K / 2) >= (int64_t(1) << 32) || w->K > kW4a4MaxK)
      return NVFP4_ERR_UNSUPPORTED;
    if (use_scratch) {
      if (need > nvfp4::scratch_capacity()) return NVFP4_ERR_WORKSPACE;  // beyond the scratch's fixed size
      if ((st = hip_status(nvfp4::scratch_pointer(&ws))) != NVFP4_OK) return st;
      ws_bytes = nvfp4::scratch_capacity();
    }
    if (!ws || ws_bytes < need_act) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(ws)) return NVFP4_ERR_ALIGNMENT;
    uint8_t* codes = static_cast<uint8_t*>(ws);
    uint8_t* scales = codes + align_up(size_t(M) * size_t(w->K / 2), 256);
    // split-K partials after the activations, when the shape takes them and
    // the workspace holds them (else one launch over all of K)
    float* partials = need > need_act && ws_bytes >= need ? reinterpret_cast<float*>(codes + need_act) : nullptr;
    st = hip_status(nvfp4::launch_quantize(a, M, w->K, lda, g_act, codes, scales, stream));
    if (st == NVFP4_OK)
      st = hip_status(
          nvfp4::launch_w4a4(codes, scales, M, w->data, w->N, w->K, alpha_w4a4, out, ldo, partials, stream));
  }
  if (st == NVFP4_OK && route_taken) *route_taken = route;
  return st;
}

}  // namespace

nvfp4_status nvfp4_linear(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* g_act,
                          const float* alpha_w4a16, const float* alpha_w4a4, void* out, int64_t ldo, void* ws,
                          size_t ws_bytes, int* route_taken, hipStream_t stream) {
  return linear_impl(a, M, lda, w, g_act, alpha_w4a16, alpha_w4a4, out, ldo, ws, ws_bytes, false, route_taken,
                     stream);
}

nvfp4_status nvfp4_linear_noalloc(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* g_act,
                                  const float* alpha_w4a16, const float* alpha_w4a4, void* out, int64_t ldo,
                                  int* route_taken, hipStream_t stream) {
  return linear_impl(a, M, lda, w, g_act, alpha_w4a16, alpha_w4a4, out, ldo, nullptr, 0, true, route_taken,
                     stream);
}

}  // extern "C"

namespace {

nvfp4_status moe_shape(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  if (T < 0 || K <= 0 || I <= 0) return NVFP4_ERR_INVALID_SHAPE;
  if (top_k < 1 || E < 1 || E > 1024) return NVFP4_ERR_INVALID_ARGUMENT;
  if (K % 16 != 0 || I % 16 != 0) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 256 != 0 || I % 256 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (K > (1 << 20) || I > (1 << 20) || T > kInt32Max || top_k > 1024) return NVFP4_ERR_UNSUPPORTED;
  if (T * top_k > kInt32Max || T * top_k / 256 + E > 65535) return NVFP4_ERR_UNSUPPORTED;
  // 32-bit byte offsets into the quantized x and h
  if (T * (K / 2) >= (int64_t(1) << 32) || T * top_k * (I / 2) >= (int64_t(1) << 32)) return NVFP4_ERR_UNSUPPORTED;
  if (E * 2 * I > kInt32Max - 15 || E * K > kInt32Max - 15) return NVFP4_ERR_UNSUPPORTED;
  // 32-bit byte offsets within one expert's prepared gate_up and down weights
  if (2 * I * (K / 256) * 2304 >= (int64_t(1) << 32)) return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_moe_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  if (moe_shape(T, top_k, E, K, I) != NVFP4_OK) return 0;
  return size_t(nvfp4::moe_layout(T, top_k, E, K, I).total);
}

nvfp4_status nvfp4_moe_workspace_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                        nvfp4_moe_layout* out) {
  if (!out) return NVFP4_ERR_INVALID_ARGUMENT;
  const nvfp4_status st = moe_shape(T, top_k, E, K, I);
  if (st != NVFP4_OK) return st;
  const nvfp4::MoeLayout L = nvfp4::moe_layout(T, top_k, E, K, I);
  out->x_codes = L.x_codes;
  out->x_scales = L.x_scales;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->tiles = L.tiles;
  out->sorted = L.sorted;
  out->h_codes = L.h_codes;
  out->h_scales = L.h_scales;
  out->inv = L.inv;
  out->ys = L.ys;
  out->max_tiles = L.max_tiles;
  out->total_bytes = L.total;
  return NVFP4_OK;
}

nvfp4_status nvfp4_moe_w4a4(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                            int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up,
                            const nvfp4_weight* down, const float* g1, const float* g2, const float* alpha_gu,
                            const float* alpha_dn, void* out, int64_t ldo, void* ws, size_t ws_bytes,
                            float* h_amax, hipStream_t stream) {
  if (!gate_up || !down) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(gate_up);
  if (st != NVFP4_OK) return st;
  if ((st = check_weight(down)) != NVFP4_OK) return st;
  const int64_t K = gate_up->K;
  if ((st = moe_shape(T, top_k, E, K, I)) != NVFP4_OK) return st;
  if (gate_up->N != E * 2 * I || down->N != E * K || down->K != I) return NVFP4_ERR_INVALID_SHAPE;
  if (!g1 || !g2 || !alpha_gu || !alpha_dn) return NVFP4_ERR_INVALID_ARGUMENT;
  if (T == 0) return NVFP4_OK;  // x, ids, out and ws may be null
  if (!topk_ids || !topk_w || !out) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((st = check_bf16_input(x, T, K, ldx)) != NVFP4_OK) return st;
  if (ldo < K) return NVFP4_ERR_INVALID_SHAPE;
  if (T > 0 && ldo > (INT64_MAX / 2) / T) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(out) || ldo % 8 != 0) return NVFP4_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(topk_ids) & 3u) || (reinterpret_cast<uintptr_t>(topk_w) & 3u) ||
      (reinterpret_cast<uintptr_t>(alpha_gu) & 3u) || (reinterpret_cast<uintptr_t>(alpha_dn) & 3u) ||
      (reinterpret_cast<uintptr_t>(h_amax) & 3u))
    return NVFP4_ERR_ALIGNMENT;
  if (!ws || ws_bytes < nvfp4_moe_workspace_bytes(T, top_k, E, K, I)) return NVFP4_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return NVFP4_ERR_ALIGNMENT;
  return hip_status(nvfp4::launch_moe_w4a4(x, T, ldx, topk_ids, topk_w, top_k, E, I, gate_up->data, down->data, K,
                                           g1, g2, alpha_gu, alpha_dn, out, ldo, ws, h_amax, stream));
}

}  // extern "C"

namespace {

nvfp4_status moe_w4a16_shape(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  if (T < 0 || K <= 0 || I <= 0) return NVFP4_ERR_INVALID_SHAPE;
  if (top_k < 1 || E < 1 || E > 1024) return NVFP4_ERR_INVALID_ARGUMENT;
  if (K % 16 != 0 || I % 16 != 0) return NVFP4_ERR_INVALID_SHAPE;
  if (K % 256 != 0 || I % 256 != 0) return NVFP4_ERR_UNSUPPORTED;
  // at most 8 steps per wave over 8 waves
  if (K > 64 * 256 || I > 64 * 256 || T > kInt32Max || top_k > 1024) return NVFP4_ERR_UNSUPPORTED;
  const int64_t P = T * top_k;
  if (P > kInt32Max) return NVFP4_ERR_UNSUPPORTED;
  // one workgroup per (entry, 16-row tile); 32-bit offsets into h
  const int64_t entries = std::min<int64_t>(P / nvfp4::kW4A16Rows + E, P);
  if (entries * (std::max(K, I) / 16) > kInt32Max) return NVFP4_ERR_UNSUPPORTED;
  if (P * I * 2 > (int64_t(1) << 31) - 4096) return NVFP4_ERR_UNSUPPORTED;
  if (E * 2 * I > kInt32Max - 15 || E * K > kInt32Max - 15) return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_moe_w4a16_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I) {
  if (moe_w4a16_shape(T, top_k, E, K, I) != NVFP4_OK) return 0;
  return size_t(nvfp4::moe_w4a16_layout(T, top_k, E, K, I).total);
}

nvfp4_status nvfp4_moe_w4a16_workspace_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                              nvfp4_moe_w4a16_layout* out) {
  if (!out) return NVFP4_ERR_INVALID_ARGUMENT;
  const nvfp4_status st = moe_w4a16_shape(T, top_k, E, K, I);
  if (st != NVFP4_OK) return st;
  const nvfp4::MoeW4A16Layout L = nvfp4::moe_w4a16_layout(T, top_k, E, K, I);
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->tiles = L.tiles;
  out->sorted = L.sorted;
  out->inv = L.inv;
  out->h = L.h;
  out->ys = L.ys;
  out->max_tiles = L.max_tiles;
  out->total_bytes = L.total;
  return NVFP4_OK;
}

nvfp4_status nvfp4_moe_w4a16(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                             int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up,
                             const nvfp4_weight* down, const float* alpha_gu, const float* alpha_dn, void* out,
                             int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!gate_up || !down) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(gate_up);
  if (st != NVFP4_OK) return st;
  if ((st = check_weight(down)) != NVFP4_OK) return st;
  const int64_t K = gate_up->K;
  if ((st = moe_w4a16_shape(T, top_k, E, K, I)) != NVFP4_OK) return st;
  if (gate_up->N != E * 2 * I || down->N != E * K || down->K != I) return NVFP4_ERR_INVALID_SHAPE;
  if (!alpha_gu || !alpha_dn) return NVFP4_ERR_INVALID_ARGUMENT;
  if (T == 0) return NVFP4_OK;  // x, ids, out and ws may be null
  if (!topk_ids || !topk_w || !out) return NVFP4_ERR_INVALID_ARGUMENT;
  if ((st = check_bf16_input(x, T, K, ldx)) != NVFP4_OK) return st;
  if ((T - 1) * ldx * 2 + 2 * K > (int64_t(1) << 31) - 4096) return NVFP4_ERR_UNSUPPORTED;  // 32-bit offsets
  if (ldo < K) return NVFP4_ERR_INVALID_SHAPE;
  if (ldo > (INT64_MAX / 2) / T) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(out) || ldo % 8 != 0) return NVFP4_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(topk_ids) & 3u) || (reinterpret_cast<uintptr_t>(topk_w) & 3u) ||
      (reinterpret_cast<uintptr_t>(alpha_gu) & 3u) || (reinterpret_cast<uintptr_t>(alpha_dn) & 3u))
    return NVFP4_ERR_ALIGNMENT;
  if (!ws || ws_bytes < nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, K, I)) return NVFP4_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return NVFP4_ERR_ALIGNMENT;
  return hip_status(nvfp4::launch_moe_w4a16(x, T, ldx, topk_ids, topk_w, top_k, E, I, gate_up->data, down->data, K,
                                            alpha_gu, alpha_dn, out, ldo, ws, stream));
}

nvfp4_status nvfp4_gated_mlp_w4a4(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* gate_up,
                                  const float* alpha, const float* g2, void* h_codes, void* h_scales, float* h_amax,
                                  hipStream_t stream) {
  if (M < 0 || !alpha || !g2) return NVFP4_ERR_INVALID_ARGUMENT;
  nvfp4_status st = check_weight(gate_up);
  if (st != NVFP4_OK) return st;
  const int64_t K = gate_up->K, I = gate_up->N / 2;
  if (gate_up->N % 2 != 0 || I % 16 != 0) return NVFP4_ERR_INVALID_SHAPE;
  if (I % 256 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (M == 0 || I == 0) return NVFP4_OK;  // empty batch: buffers may be null
  if (!a_codes || !a_scales || !h_codes || !h_scales) return NVFP4_ERR_INVALID_ARGUMENT;
  if (M > kInt32Max) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(h_codes) ||
      (reinterpret_cast<uintptr_t>(h_amax) & 3u))
    return NVFP4_ERR_ALIGNMENT;
  // grid rows of 256 activation rows; 32-bit byte offsets into the codes
  if ((M + 255) / 256 * (I / 128) > kInt32Max || M * (K / 2) >= (int64_t(1) << 32) ||
      M * (I / 2) >= (int64_t(1) << 32))
    return NVFP4_ERR_UNSUPPORTED;
  // 32-bit byte offsets within the prepared gate_up weight
  if (2 * I * (K / 256) * 2304 >= (int64_t(1) << 32)) return NVFP4_ERR_UNSUPPORTED;
  return hip_status(nvfp4::launch_gated_mlp_w4a4(a_codes, a_scales, M, gate_up->data, K, I, alpha, g2, h_codes,
                                                 h_scales, h_amax, stream));
}

int nvfp4_moe_route(int64_t T, int64_t top_k, int64_t E, int has_act_globals) {
  if (!has_act_globals || E < 1) return NVFP4_ROUTE_W4A16;
  return T * top_k > g_moe_route_tpe_max.load() * E ? NVFP4_ROUTE_W4A4 : NVFP4_ROUTE_W4A16;
}

void nvfp4_set_moe_route_tokens_per_expert(int64_t tpe_max) {
  g_moe_route_tpe_max.store(std::max<int64_t>(0, std::min<int64_t>(tpe_max, int64_t(1) << 31)));
}

int64_t nvfp4_get_moe_route_tokens_per_expert(void) { return g_moe_route_tpe_max.load(); }

size_t nvfp4_moe_dispatch_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                          int has_act_globals) {
  return nvfp4_moe_route(T, top_k, E, has_act_globals) == NVFP4_ROUTE_W4A4
             ? nvfp4_moe_workspace_bytes(T, top_k, E, K, I)
             : nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, K, I);
}

nvfp4_status nvfp4_moe(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                       int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up, const nvfp4_weight* down,
                       const float* g1, const float* g2, const float* alpha_gu_w4a4, const float* alpha_dn_w4a4,
                       const float* alpha_gu_w4a16, const float* alpha_dn_w4a16, void* out, int64_t ldo, void* ws,
                       size_t ws_bytes, int* route_taken, hipStream_t stream) {
  if ((g1 == nullptr) != (g2 == nullptr)) return NVFP4_ERR_INVALID_ARGUMENT;  // both globals or neither
  const int route = nvfp4_moe_route(T, top_k, E, g1 != nullptr);
  if (route_taken) *route_taken = route;
  if (route == NVFP4_ROUTE_W4A4)
    return nvfp4_moe_w4a4(x, T, ldx, topk_ids, topk_w, top_k, E, I, gate_up, down, g1, g2, alpha_gu_w4a4,
                          alpha_dn_w4a4, out, ldo, ws, ws_bytes, nullptr, stream);
  return nvfp4_moe_w4a16(x, T, ldx, topk_ids, topk_w, top_k, E, I, gate_up, down, alpha_gu_w4a16, alpha_dn_w4a16,
                         out, ldo, ws, ws_bytes, stream);
}

nvfp4_status nvfp4_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return NVFP4_OK;
  if (!src || !sink) return NVFP4_ERR_INVALID_ARGUMENT;
  if (bytes % 16 != 0 || bytes > size_t(INT64_MAX)) return NVFP4_ERR_INVALID_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return NVFP4_ERR_ALIGNMENT;
  if (bytes / 16 > size_t(0xffffff00u)) return NVFP4_ERR_UNSUPPORTED;  // 32-bit dispatch size in threads
  return hip_status(nvfp4::launch_stream_read(src, int64_t(bytes), sink, stream));
}

}  // extern "C"
