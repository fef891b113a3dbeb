/*
 * nvfp4.h -- C ABI of the NVFP4 quantized linear for AMD Instinct MI355X (gfx950).
 *
 * Formats (FlashInfer PR #3597 "Add BF16_FP4 GEMM ... for W4A16 workloads",
 * Description, API example and review thread; FreeToken PR #737, Changes):
 *   - a weight or activation matrix [rows, K] in NVFP4 is two device buffers:
 *       codes  uint8 [rows, K/2]  two e2m1 codes per byte, even k in the low
 *                                 nibble; a code keeps its sign in bit 3 and
 *                                 its magnitude index (0, .5, 1, 1.5, 2, 3, 4,
 *                                 6) in bits 2..0;
 *       scales uint8 [rows, K/16] one OCP FP8 E4M3 block scale per 16 k,
 *                                 row-major (no swizzle);
 *     plus an fp32 per-tensor global g = 448*6 / max|x| (static for
 *     activations, from a calibration batch);
 *   - the value of element k of a row is e2m1(code) * E4M3(scale[k/16]) and
 *     the real value it stands for is that divided by g.
 *
 * Conventions shared by every call:
 *   - all tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates, frees and synchronises nothing and launches only on the given
 *     stream, so calls may be captured in a HIP graph;
 *   - bf16 tensors hold raw bfloat16 bits; scalar inputs (globals, alphas) are
 *     1-element fp32 DEVICE buffers, so no call reads device memory on the host;
 *   - every argument is validated on the host before any launch; on error the
 *     call returns a status and launches nothing; a failed launch returns
 *     NVFP4_ERR_HIP (from hipGetLastError, without synchronising);
 *   - M = 0 (or N = 0) is a successful no-op;
 *   - nothing is printed and no C++ exception crosses the ABI.
 *   - Shapes: K % 16 == 0 for the quantizer; K % 256 == 0 for the prepared
 *     weight and the linears (NVFP4_ERR_UNSUPPORTED otherwise).  Row strides (lda, ldo) count
 *     elements; bf16 inputs need 16-byte aligned base pointers and lda % 8 == 0;
 *     code / scale buffers need 16-byte aligned bases.  Outputs accept any
 *     ldo >= N and any base alignment of 2 bytes.  Sizes must fit in int32
 *     (M, N, K < 2^31 and M*K/16 < 2^31).
 *
 * Numerics (decisions every caller can rely on):
 *   - quantization decides on the exact real values amax*g/6 and |x|*g/S:
 *     nearest E4M3 scale (ties to even mantissa, saturating at 448) and
 *     nearest e2m1 magnitude (ties to even, saturating at 6); a scale that
 *     rounds to 0 gives magnitude 0 everywhere; the sign bit of x is kept;
 *   - the linears dequantize exactly, accumulate in fp32 (order unspecified
 *     for the W4A4 path; fixed for the W4A16 path), multiply by alpha, and
 *     round once to bf16 (nearest even).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARGUMENT = 1, /* null pointer where one is required, negative size */
  NVFP4_ERR_INVALID_SHAPE = 2,    /* K % 16 != 0, lda < K, ldo < N, size overflow */
  NVFP4_ERR_ALIGNMENT = 3,        /* misaligned base pointer or stride */
  NVFP4_ERR_UNSUPPORTED = 4,      /* valid NVFP4 but outside this build's kernels (K % 256, M > 64 on W4A16) */
  NVFP4_ERR_WORKSPACE = 5,        /* workspace missing or too small */
  NVFP4_ERR_HIP = 6               /* a kernel launch failed */
} nvfp4_status;

/* Layouts of a prepared weight. */
enum { NVFP4_LAYOUT_TILED = 1 };

/* Prepared weight descriptor: plain data, no heap state.  Produced by
 * nvfp4_prepare_weight; "freeing" it is the caller freeing the buffer it
 * passed as dst.  The linears read nothing but data. */
typedef struct nvfp4_weight {
  const void* data;   /* device, the tiled weight (nvfp4_prepared_weight_bytes bytes) */
  int64_t N;
  int64_t K;
  int32_t layout;     /* NVFP4_LAYOUT_TILED */
  int32_t reserved;
} nvfp4_weight;

/* Routes of the M-threshold dispatch. */
enum { NVFP4_ROUTE_W4A16 = 0, NVFP4_ROUTE_W4A4 = 1 };

/* Human-readable name of a status (static storage). */
const char* nvfp4_status_str(nvfp4_status s);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int nvfp4_version(void);

/* Hash of the sources this library was built from (16 hex digits of a
 * sha256 over its source files and this header; "unknown" when built without
 * it), so that a loader can refuse a library built from other sources.
 * Static storage. */
const char* nvfp4_build_source_hash(void);

/* ---------------------------------------------------------------------------
 * nvfp4_quantize_act -- NVFP4 quantization of bf16 rows under a static global.
 * FreeToken PR #737, Changes (the activation quant kernel of the W4A4 route,
 * split into row blocks); FlashInfer PR #3597, Description (per-16-element
 * FP8-E4M3 block scales) and API example (global (448*6)/max|x|).
 *   a      bf16 [M, K], row stride lda >= K (elements)
 *   g      device fp32[1], the global scale g > 0 (finite)
 *   codes  out, uint8 [M, K/2] contiguous
 *   scales out, uint8 [M, K/16] contiguous
 * Per 16-element block: scale = E4M3(amax*g/6), code_i = sign | e2m1(|x_i|*g/S).
 * Works on weights as well (quantizing a bf16 weight with its own global).
 * Errors: INVALID_ARGUMENT (null), INVALID_SHAPE (K % 16, lda < K),
 * ALIGNMENT (a, codes not 16-byte aligned, lda % 8), HIP.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_act(const void* a, int64_t M, int64_t K, int64_t lda, const float* g,
                                void* codes, void* scales, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_global_scale -- calibration helper: g = fp32(448*6 / max|x|) of a bf16
 * matrix, with IEEE fp32 division (FlashInfer PR #3597, API example:
 * g_w = (448 * 6) / w.float().abs().max()).  0 for an all-zero matrix.
 *   x      bf16 [rows, cols], row stride ld; cols % 8 == 0
 *   g_out  device fp32[1]; also used as the reduction's scratch word
 * Three launches on the stream (clear, reduce, divide).
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_global_scale(const void* x, int64_t rows, int64_t cols, int64_t ld, float* g_out,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_alpha -- alpha = fp32(1 / (g_w * g_a)), the product and quotient in
 * double as the pages' Python computes it (FlashInfer PR #3597, API example:
 * alpha = 1.0 / g_w.item() stored as fp32).  g_a may be NULL (W4A16 alpha
 * 1/g_w).  One single-thread launch.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_alpha(const float* g_w, const float* g_a, float* alpha_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_prepare_weight -- re-tile a canonical NVFP4 weight once into the
 * layout both linears read (FlashInfer PR #3597, API: prepare_bf16_fp4_weights
 * runs once per weight so the GEMM dequantizes fast; FreeToken PR #737,
 * Changes: one weight copy serves the W4A16 and W4A4 linears).
 *   codes   device uint8 [N, K/2], row-major, 8-byte aligned
 *   scales  device uint8 [N, K/16], row-major
 *   dst     device buffer of at least nvfp4_prepared_weight_bytes(N, K) bytes,
 *           16-byte aligned, owned by the caller; after the call's work has
 *           run on the stream the canonical codes/scales may be freed
 *   out     host pointer to the descriptor to fill
 * Tiled layout: ceil(N/16) * (K/256) units of 2304 bytes; unit (t, s) at byte
 * (t * K/256 + s) * 2304 covers rows 16t..16t+15 (rows >= N are zero) and
 * k in [256s, 256s + 256).  With lane l = r + 16q (r = row in the tile,
 * q = 0..3) owning the 16-k groups 4p + q (p = 0..3) of its row:
 *   unit bytes [16l, 16l+16)         canonical code bytes of groups q, 4+q
 *   unit bytes [1024+16l, +16)       canonical code bytes of groups 8+q, 12+q
 *   unit bytes [2048+4l, +4)         scale bytes of groups q, 4+q, 8+q, 12+q
 * One launch on the stream.  nvfp4_prepared_weight_bytes returns 0 for an
 * invalid shape.
 * Errors: INVALID_ARGUMENT (null), INVALID_SHAPE (K % 16, N < 0),
 * UNSUPPORTED (K % 256), WORKSPACE (dst_bytes too small), ALIGNMENT, HIP.
 * ------------------------------------------------------------------------- */
size_t nvfp4_prepared_weight_bytes(int64_t N, int64_t K);
nvfp4_status nvfp4_prepare_weight(const void* codes, const void* scales, int64_t N, int64_t K, void* dst,
                                  size_t dst_bytes, nvfp4_weight* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Interop with the 128x4-swizzled block-scale layout that checkpoints and
 * NVIDIA's block-scaled GEMMs use (the FreeToken PR #737 page, Changes: the
 * linears keep the checkpoint's codes with 128x4-swizzled scales, and the
 * activation quant kernel can write that layout; FlashInfer PR #3597, API:
 * weights prepared with the 128x4 scale-factor layout).  The pages name the
 * layout without its index map; this library takes the public one: the
 * [rows, K/16] scale matrix is padded with zeros to a multiple of 128 rows and
 * 4 columns and stored as 512-byte blocks of 128 rows x 4 columns, row-major
 * over the blocks; inside a block, scale (r, c) sits at byte
 * 16 (r % 32) + 4 ((r / 32) % 4) + c % 4.
 * nvfp4_swizzled_scales_bytes(rows, K) = roundup(rows, 128) * roundup(K/16, 4),
 * 0 for an invalid shape (rows < 0, K <= 0, K % 16).
 *
 * nvfp4_quantize_act_swizzled: nvfp4_quantize_act with the scales written in
 * that layout, padding included (zeros), into scales (>= scales_bytes =
 * nvfp4_swizzled_scales_bytes(M, K) bytes; WORKSPACE if smaller).  Codes and
 * scale values are those of nvfp4_quantize_act, bit for bit.  Other
 * arguments and errors as nvfp4_quantize_act.
 *
 * nvfp4_prepare_weight_swizzled: nvfp4_prepare_weight from row-major codes
 * [N, K/2] and swizzled scales (scales_bytes >= nvfp4_swizzled_scales_bytes(N,
 * K), else WORKSPACE); the result is byte for byte the one nvfp4_prepare_weight
 * makes from the same scales in row-major order.  Errors as
 * nvfp4_prepare_weight.
 * ------------------------------------------------------------------------- */
size_t nvfp4_swizzled_scales_bytes(int64_t rows, int64_t K);

/* nvfp4_fused_weight_global -- the one weight global of a fused weight (say
 * q|k|v or gate|up stored as one [N, K] matrix) whose parts were quantized
 * under their own globals: the largest per-part global, with the block
 * scales unchanged (the FreeToken PR #737 page, Changes, which also warns at
 * load time when the parts' globals differ by more than 5 %).  A host call on
 * host memory, no launch.
 *   g_parts  host fp32[n_parts], each finite and > 0
 *   g_out    host fp32: max of g_parts
 *   warn     host int32 or NULL: 1 when max > 1.05 * min (in double), else 0
 * Errors: INVALID_ARGUMENT (null, n_parts <= 0, a global not finite or <= 0). */
nvfp4_status nvfp4_fused_weight_global(const float* g_parts, int64_t n_parts, float* g_out, int32_t* warn);
nvfp4_status nvfp4_quantize_act_swizzled(const void* a, int64_t M, int64_t K, int64_t lda, const float* g,
                                         void* codes, void* scales, size_t scales_bytes, hipStream_t stream);
nvfp4_status nvfp4_prepare_weight_swizzled(const void* codes, const void* scales, size_t scales_bytes, int64_t N,
                                           int64_t K, void* dst, size_t dst_bytes, nvfp4_weight* out,
                                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_linear_w4a16 -- out = bf16((a @ dequant(W).T) * alpha), fp32
 * accumulation (FlashInfer PR #3597, Description), for decode-sized M <= 64
 * (FreeToken PR #737, Changes: small-batch kernels on the same weight; its
 * Results keep a W4A16 tier to about 48 tokens).  Up to 16 tokens several
 * schedules; 17..64 tokens the shared schedule with up to four 16-token
 * groups on each dequantized weight fragment.
 *   a      bf16 [M, K], lda >= K
 *   w      prepared weight descriptor (host pointer)
 *   alpha  device fp32[1] (1/g_w)
 *   out    bf16 [M, N], ldo >= N
 * One launch, no workspace.  Deterministic: the fp32 sum order depends only
 * on (M, N, K).
 * Errors: as above; UNSUPPORTED for M > 64, or when a's last row ends 2^31 -
 * 4096 bytes or more past its first element ((M-1)*lda*2 + 2*K; the kernels
 * address the activations with 32-bit offsets).
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_linear_w4a16(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* alpha,
                                void* out, int64_t ldo, hipStream_t stream);

/* Same with an explicit schedule (for tests and tuning):
 *   schedule 0     the default for (M, N, K); the other arguments are ignored
 *   schedule 1     split: one workgroup per 16-row tile whose ksplit (1..16)
 *                  waves split K into contiguous runs of 256-k steps
 *   schedule 2     shared: one workgroup per 8 tiles (16 on weights of at
 *                  least 12 tiles per CU) over all of K, the activations
 *                  streamed through LDS in chunks of chunk_steps 256-k steps;
 *                  needs R * min(chunk_steps, K/256) <= 64 with R = M
 *                  up to 16 tokens and 16 * ceil(M/16) above;
 *                  the only schedule for M > 16 (INVALID_ARGUMENT otherwise)
 *   schedule 3     split with interleaved steps (wave w takes steps w,
 *                  w + waves, ...); needs ceil(K/256 / ksplit) <= 8.  Here
 *                  chunk_steps is the tiles per workgroup: 0 or 1, or 2
 *                  (each step's activation operands serve both tiles; at
 *                  most 8 waves)
 *   schedule 4     dot: schedule 3's work split with the products on the
 *                  VALU (bf16 dot products, activations broadcast across
 *                  lanes); needs M <= 4 and ceil(K/256 / ksplit) <= 8
 * cache_policy (schedule 4 only; 0 elsewhere, INVALID_ARGUMENT otherwise):
 *                  0 the default: weight loads nontemporal (streamed without
 *                  keeping them in the caches), activation loads default;
 *                  1 weight loads default; 2 activation loads nontemporal
 *                  too.  Same results; a tactic measured in a sequence of
 *                  kernels (FreeToken PR #737, Changes, notes that a cache
 *                  hint on the weights can help a linear alone and hurt the
 *                  kernels after it).
 * Other values return INVALID_ARGUMENT.  The result bits depend on (M, N, K)
 * and the schedule. */
nvfp4_status nvfp4_linear_w4a16_ex(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w,
                                   const float* alpha, void* out, int64_t ldo, int schedule, int ksplit,
                                   int chunk_steps, int cache_policy, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_linear_w4a4 -- out = bf16((dequant(A) @ dequant(W).T) * alpha) on
 * NVFP4 activations, alpha = 1/(g_w * g_a) (FreeToken PR #737, Changes:
 * prefill runs W4A4 GEMMs on NVFP4 activations; FreeToken PR #736, Changes:
 * the same product inside the MoE experts).
 *   a_codes, a_scales  uint8 [M, K/2], [M, K/16] contiguous (nvfp4_quantize_act output)
 *   w                  prepared weight descriptor
 *   alpha              device fp32[1]
 *   out                bf16 [M, N], ldo >= N
 * One launch over all of K, no workspace: 256 x 256 output tiles, or for a
 * batch of at most 128 rows, 256 weight rows per workgroup over all M rows.
 * K above 2^24 returns UNSUPPORTED (the kernels' 32-bit weight offsets).
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_linear_w4a4(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* w,
                               const float* alpha, void* out, int64_t ldo, hipStream_t stream);

/* nvfp4_linear_w4a4 with a workspace for a split of K across workgroups
 * (split-K).  A small batch on a weight of a few thousand rows has few
 * output tiles of 256 weight rows (N = 8704 has 34), and one workgroup per
 * tile leaves most CUs idle while each works through all of K.  When the
 * tiles fill at most half the CUs, K is split into S ranges of whole 256-k
 * units (S <= 16, at least two units each); tile x range workgroups store
 * fp32 partial tiles in ws, and a second launch adds the ranges' partials in
 * range order (fixed fp32 order: deterministic), scales by alpha and rounds
 * once to bf16.  The sum order differs from the one-launch call's, so the
 * bits can differ from nvfp4_linear_w4a4's (both meet the same bar).
 *   nvfp4_linear_w4a4_workspace_bytes: S * M * N * 4 bytes (256-byte
 *   aligned) when the shape splits on the current device, else 0 (then ws
 *   may be NULL and the call is nvfp4_linear_w4a4's one launch).  S keeps the
 *   partials within 48 MiB and, with nvfp4_linear's quantized activations,
 *   within NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES.
 *   ws, ws_bytes  device workspace, 16-byte aligned, >= the bytes above
 * Errors: as nvfp4_linear_w4a4, plus WORKSPACE (ws missing or too small) and
 * ALIGNMENT (ws). */
size_t nvfp4_linear_w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_linear_w4a4_ws(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* w,
                                  const float* alpha, void* out, int64_t ldo, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * M-threshold dispatch (FreeToken PR #737, Changes: W4A4 for prefill on
 * checkpoints with static activation scales, W4A16 kernels for batches up to
 * a threshold T, 8 or 16 there).
 *   nvfp4_route: pure; W4A4 iff has_act_global && M > M*; else W4A16.
 *   nvfp4_set_route_m_max / get: M* (default 16: from 17 rows on, quantize
 *   + W4A4 beats the W4A16 kernels on the large fused weight N = 62080,
 *   K = 5120 on MI355X, and on N = 3584, 8704 and 43008 (K = 5120); on
 *   N = 14336 and 28672 W4A16 stays ahead up to about 24 and 56 rows.
 *   Values above 64 are clamped to 64, the W4A16 kernels' limit, and a
 *   missing activation global with M > 64 is UNSUPPORTED).
 * ------------------------------------------------------------------------- */
int nvfp4_route(int64_t M, int64_t N, int64_t K, int has_act_global);
void nvfp4_set_route_m_max(int64_t m_max);
int64_t nvfp4_get_route_m_max(void);

/* Workspace nvfp4_linear needs on the W4A4 route: M*K/2 + M*K/16 bytes
 * (256-byte aligned parts) for the quantized activations, then
 * nvfp4_linear_w4a4_workspace_bytes(M, N, K) for the split-K partials (the
 * W4A4 route runs nvfp4_linear_w4a4_ws's kernels); the W4A16 route uses none.
 * The partials make the total larger for some small M than for a large one
 * (N = 8704, K = 5120: 42.7 MB at M = 256, 23.6 MB at M = 8192).  A workspace
 * that holds the activations but not the partials runs the one-launch kernel
 * instead (nvfp4_linear_w4a4's bits); only less than the activations is a
 * WORKSPACE error. */
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* ---------------------------------------------------------------------------
 * nvfp4_linear -- the dispatched linear: W4A16 on bf16 a when M <= M* (or no
 * activation global), else quantize a under g_act into the workspace and run
 * W4A4.  The routes give different numerics, so the route taken is returned.
 *   g_act         device fp32[1] or NULL (W4A16 only)
 *   alpha_w4a16   device fp32[1], 1/g_w
 *   alpha_w4a4    device fp32[1], 1/(g_w g_act) (may be NULL when g_act is)
 *   ws, ws_bytes  device workspace, >= nvfp4_linear_workspace_bytes(M, N, K)
 *                 on the W4A4 route for the split-K kernels, at least the
 *                 activations' part for the one-launch kernel (may be NULL
 *                 on the W4A16 route)
 *   route_taken   host int out (NVFP4_ROUTE_*), may be NULL
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_linear(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* g_act,
                          const float* alpha_w4a16, const float* alpha_w4a4, void* out, int64_t ldo, void* ws,
                          size_t ws_bytes, int* route_taken, hipStream_t stream);

/* Size of the library's own scratch on each GPU, used by nvfp4_linear_noalloc
 * for the W4A4 route's quantized activations and split-K partials:
 * nvfp4_linear_workspace_bytes(M, N, K) must not exceed it (M = 8192 at
 * K = 5120 needs 23.6 MB; the split-K partials are sized to fit beside the
 * activations). */
#define NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)64 << 20)

/* nvfp4_linear without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing and frees
 * nothing.  On the W4A4 route the quantized activations (and the split-K
 * partials) go to a scratch array the library holds on each GPU (a device global of
 * NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES, kept until the process ends);
 * the W4A16 route needs none.  The caller still passes inputs and outputs.
 *   Arguments, routes, numerics and errors as nvfp4_linear with a workspace
 *   of nvfp4_linear_workspace_bytes(M, N, K) (the same kernels, the same
 *   bits), plus WORKSPACE when nvfp4_linear_workspace_bytes(M, N, K)
 *   exceeds NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES on the W4A4 route
 *   (checked before any launch).
 *   Every call on one GPU shares that GPU's scratch, so calls that overlap in
 *   time on one GPU (on different streams) race and must not be issued; calls
 *   on one stream are ordered and safe.  The first call on each device looks
 *   up the scratch's device address (hipGetSymbolAddress, not a stream
 *   operation); make that first call outside graph capture.  Nothing in the
 *   scratch needs clearing: each call overwrites what it reads. */
nvfp4_status nvfp4_linear_noalloc(const void* a, int64_t M, int64_t lda, const nvfp4_weight* w, const float* g_act,
                                  const float* alpha_w4a16, const float* alpha_w4a4, void* out, int64_t ldo,
                                  int* route_taken, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * NVFP4 MoE expert layer, W4A4 on both GEMMs (FreeToken PR #736, Changes and
 * Results: both expert GEMMs take NVFP4 activations with static input scales,
 * the gate_up epilogue applies the gated activation and quantizes its output
 * to NVFP4, the down epilogue applies the routing weight and sums the routes;
 * FreeToken PR #733, Changes: the layer runs align, gate_up, activation, down
 * and the route sum).  For token t, route r < top_k, e = topk_ids[t, r]:
 *   z      = alpha_gu[e] * (dequant(q(x_t; g1)) @ dequant(W_gu[e]).T)   [2I]
 *   h      = SiLU(z[0:I]) * z[I:2I], SiLU(v) = v / (1 + exp(-v)), fp32
 *   y      = alpha_dn[e] * (dequant(q(h; g2)) @ dequant(W_dn[e]).T)     [K]
 *   out[t] = bf16(sum_r topk_w[t, r] * y_r), the sum in fp32
 * q(.; g) is the NVFP4 quantization of nvfp4_quantize_act (h is never rounded
 * to bf16).  Rows [0, I) of an expert's gate_up weight are the gate, [I, 2I)
 * the up projection.  A pair whose id lies outside [0, E) is skipped: it adds
 * nothing to its token's sum (expert-parallel callers pass -1 for experts they
 * do not hold).
 *   x          bf16 [T, K], row stride ldx (>= K, multiple of 8), 16-byte aligned
 *   topk_ids   device int32 [T, top_k]; topk_w device fp32 [T, top_k]
 *   gate_up    prepared weight of the E stacked [2I, K] banks (N = E*2I, K)
 *   down       prepared weight of the E stacked [K, I] banks (N = E*K, K = I)
 *   g1, g2     device fp32[1]: static globals of x and of h
 *   alpha_gu, alpha_dn  device fp32[E]: 1/(g_gu[e] g1), 1/(g_dn[e] g2)
 *   out        bf16 [T, K], row stride ldo (multiple of 8), 16-byte aligned
 *   ws         device workspace >= nvfp4_moe_workspace_bytes, 256-byte aligned
 *   h_amax     device fp32[1] or NULL: receives max |h| over the pairs (the
 *              calibration of a static g2 runs the layer on a calibration
 *              batch with any g2 and sets g2 = 2688 / h_amax)
 * Needs K % 256 == 0, I % 256 == 0, 1 <= E <= 1024, T*top_k < 2^31 and
 * T*top_k/256 + E <= 65535.  Seven launches on the stream, no host sync.  The
 * down GEMM stores each pair's routing-weighted y in fp32 by slot and a last
 * launch adds a token's routes in the order r = 0, 1, ...: the outputs are
 * the same bits on every call.
 * After the call the workspace holds, at the offsets nvfp4_moe_workspace_layout
 * reports, the align results and h (for inspection):
 *   sorted     int32 [T*top_k]: pair index t*top_k + r at each slot, pairs
 *              grouped by expert, in pair order within an expert
 *   offsets    int32 [E + 1]: first slot of each expert, [E] = pairs kept
 *   tiles      int32 [max_tiles, 4]: (expert, first slot, rows, 0) of each
 *              tile of up to 256 slots, rows == 0 past the last tile
 *   h_codes    uint8 [T*top_k, I/2], h_scales uint8 [T*top_k, I/16], by slot
 *   inv        int32 [T*top_k]: slot of pair t*top_k + r, -1 for a skipped pair
 * Errors: INVALID_ARGUMENT (null, top_k < 1, E out of range), INVALID_SHAPE
 * (descriptor shapes disagree, strides), UNSUPPORTED (K or I % 256, sizes
 * beyond the limits), WORKSPACE, ALIGNMENT, HIP.
 * ------------------------------------------------------------------------- */
typedef struct nvfp4_moe_layout {
  int64_t x_codes, x_scales;  /* quantized x [T, K/2], [T, K/16] */
  int64_t counts;             /* int32 [chunks, E] scratch */
  int64_t offsets;            /* int32 [E + 1] */
  int64_t tiles;              /* int32 [max_tiles, 4] */
  int64_t sorted;             /* int32 [T*top_k] */
  int64_t h_codes, h_scales;  /* uint8 [T*top_k, I/2], [T*top_k, I/16] */
  int64_t inv;                /* int32 [T*top_k]: slot of each pair, -1 if skipped */
  int64_t ys;                 /* fp32 [T*top_k, K]: routing-weighted y by slot */
  int64_t max_tiles;
  int64_t total_bytes;
} nvfp4_moe_layout;

size_t nvfp4_moe_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I);
nvfp4_status nvfp4_moe_workspace_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                        nvfp4_moe_layout* out);
nvfp4_status nvfp4_moe_w4a4(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                            int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up,
                            const nvfp4_weight* down, const float* g1, const float* g2, const float* alpha_gu,
                            const float* alpha_dn, void* out, int64_t ldo, void* ws, size_t ws_bytes,
                            float* h_amax, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_moe_w4a16 -- the same expert layer with W4A16 on both GEMMs (bf16
 * activations, NVFP4 banks), for decode-sized batches: the pages' layer keeps
 * W4A16 below 4 tokens per expert and for decode, on the same banks as the
 * W4A4 path (FreeToken PR #736, Changes; FreeToken PR #733, Changes: align,
 * gate_up, activation, down, sum).  For token t, route r, e = topk_ids[t, r]:
 *   z      = alpha_gu[e] * (x_t @ dequant(W_gu[e]).T)          [2I], fp32 sums
 *   h      = bf16(SiLU(z[0:I]) * z[I:2I]), SiLU in fp32
 *   y      = alpha_dn[e] * (h @ dequant(W_dn[e]).T)             [K], fp32 sums
 *   out[t] = bf16(sum_r topk_w[t, r] * y_r), the sum in fp32, r = 0, 1, ...
 * alpha_gu[e] = 1/g_gu[e], alpha_dn[e] = 1/g_dn[e] (no activation globals).
 * A pair whose id lies outside [0, E) is skipped.  Arguments as
 * nvfp4_moe_w4a4 without g1, g2 and h_amax; ws >= nvfp4_moe_w4a16_workspace_bytes.
 * The align cuts each expert's pairs into entries of up to 16; both GEMMs run
 * one workgroup per (entry, 16-row tile of the expert's weight), so a call
 * reads the banks of the experts it routes to, each once per 16 of its pairs
 * (an entry of one or two pairs on VALU dot products, a larger one on the
 * MFMA).  A pair's fp32 sum order follows its entry's size, so a token's
 * output bits may change (within fp32 rounding) with the number of other
 * pairs routed to its experts; for given inputs the outputs are the same.
 * Up to five launches, no host sync; the outputs are the same bits on every
 * call.  After the call the workspace holds, at the offsets
 * nvfp4_moe_w4a16_workspace_layout reports: sorted, offsets, inv (as for
 * nvfp4_moe_w4a4), tiles (entries of up to 16 slots) and h (bf16 [T*top_k, I]
 * by slot).
 * Few pairs (T*top_k <= NVFP4_MOE_W4A16_DIRECT_PAIRS, top_k <= 16, I <= 2048):
 * every pair is its own entry and the layer runs in two launches without the
 * align -- gate_up per pair, storing h at the pair index t*top_k + r (a
 * skipped pair's row is not written), then down and the route sum together,
 * one wave per route adding the token's routes in the order r = 0, 1, ... in
 * fp32.  sorted, offsets, tiles and inv are then not written.
 * Needs K % 256 == 0, I % 256 == 0, K and I <= 16384, 1 <= E <= 1024,
 * T*top_k < 2^31, h below 2^31 bytes and x's last row ending below 2^31 bytes.
 * Errors as nvfp4_moe_w4a4.
 * ------------------------------------------------------------------------- */
#define NVFP4_MOE_W4A16_DIRECT_PAIRS 64

typedef struct nvfp4_moe_w4a16_layout {
  int64_t counts, offsets, tiles, sorted, inv;  /* as nvfp4_moe_layout */
  int64_t h;                                    /* bf16 [T*top_k, I] by slot */
  int64_t ys;                                   /* fp32 [T*top_k, K]: routing-weighted y by slot */
  int64_t max_tiles;
  int64_t total_bytes;
} nvfp4_moe_w4a16_layout;

size_t nvfp4_moe_w4a16_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I);
nvfp4_status nvfp4_moe_w4a16_workspace_layout(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                              nvfp4_moe_w4a16_layout* out);
nvfp4_status nvfp4_moe_w4a16(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                             int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up,
                             const nvfp4_weight* down, const float* alpha_gu, const float* alpha_dn, void* out,
                             int64_t ldo, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_gated_mlp_w4a4 -- the first GEMM of a gated MLP on NVFP4 activations
 * with the MoE gate_up epilogue (FreeToken PR #736, Changes: the gate_up GEMM
 * applies the gated activation and quantizes its output to NVFP4, so the next
 * GEMM's input needs no separate pass), for a dense batch:
 *   z      = alpha * (dequant(A) @ dequant(W_gu).T)      [M, 2I], fp32 sums
 *   h      = SiLU(z[:, 0:I]) * z[:, I:2I]                  fp32
 *   h_codes, h_scales = nvfp4_quantize_act(h; g2)          [M, I/2], [M, I/16]
 * Rows [0, I) of the weight are the gate, [I, 2I) the up projection; the
 * outputs feed nvfp4_linear_w4a4 (the down projection) directly.
 *   a_codes, a_scales  uint8 [M, K/2], [M, K/16] contiguous, 16-byte aligned
 *   gate_up            prepared weight [2I, K]; I % 256 == 0
 *   alpha              device fp32[1]: 1/(g_gu g_a); g2 device fp32[1]
 *   h_codes, h_scales  uint8 [M, I/2] (16-byte aligned), [M, I/16], contiguous
 *   h_amax             device fp32[1] or NULL: receives max |h| (calibration of g2)
 * One launch (two with h_amax), no workspace, no host sync.  The h decisions
 * are exact comparisons on the fp32 h (as in nvfp4_moe_w4a4).
 * Errors: INVALID_ARGUMENT (nulls), INVALID_SHAPE (odd N, I % 16), UNSUPPORTED
 * (I % 256, offsets past 2^32 bytes), ALIGNMENT, HIP.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_gated_mlp_w4a4(const void* a_codes, const void* a_scales, int64_t M, const nvfp4_weight* gate_up,
                                  const float* alpha, const float* g2, void* h_codes, void* h_scales, float* h_amax,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Tokens-per-expert dispatch between the two MoE layers (FreeToken PR #736,
 * Changes: W4A4 prefill from 4 tokens per expert on checkpoints whose experts
 * carry static input scales, W4A16 below and for decode).
 *   nvfp4_moe_route: pure; W4A4 iff has_act_globals && T*top_k > tpe * E,
 *     else W4A16.  tpe (tokens per expert) defaults to 14, the measured
 *     crossover on MI355X at E = 128, top-8, K = 2048, I = 768 (W4A16 108 us
 *     against W4A4 123 us at T = 192, 12 tokens per expert; 129 against 121
 *     at T = 256, 16 per expert); set it with
 *     nvfp4_set_moe_route_tokens_per_expert (negative values give 0).
 *   nvfp4_moe_dispatch_workspace_bytes: the workspace of the route taken.
 *   nvfp4_moe: runs the route taken, reports it in *route_taken (may be
 *     NULL).  g1 and g2 are both given (W4A4 possible) or both NULL (W4A16
 *     only; INVALID_ARGUMENT if only one is).  The W4A4 route takes
 *     alpha_*_w4a4 = 1/(g_e g1), 1/(g_e g2); the W4A16 route alpha_*_w4a16 =
 *     1/g_e.  Other arguments and errors as the layer taken.  The two layers'
 *     numerics differ (NVFP4 vs bf16 activations).
 * ------------------------------------------------------------------------- */
int nvfp4_moe_route(int64_t T, int64_t top_k, int64_t E, int has_act_globals);
void nvfp4_set_moe_route_tokens_per_expert(int64_t tpe_max);
int64_t nvfp4_get_moe_route_tokens_per_expert(void);
size_t nvfp4_moe_dispatch_workspace_bytes(int64_t T, int64_t top_k, int64_t E, int64_t K, int64_t I,
                                          int has_act_globals);
nvfp4_status nvfp4_moe(const void* x, int64_t T, int64_t ldx, const int32_t* topk_ids, const float* topk_w,
                       int64_t top_k, int64_t E, int64_t I, const nvfp4_weight* gate_up, const nvfp4_weight* down,
                       const float* g1, const float* g2, const float* alpha_gu_w4a4, const float* alpha_dn_w4a4,
                       const float* alpha_gu_w4a16, const float* alpha_dn_w4a16, void* out, int64_t ldo, void* ws,
                       size_t ws_bytes, int* route_taken, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * nvfp4_stream_read -- a measurement aid, not part of the NVFP4 method: reads
 * `bytes` of device memory once (one 16-byte nontemporal load per thread, the
 * way the W4A16 kernels read their weight units) and computes nothing from the
 * data, except that a 4-byte value is written to *sink in the rare case the
 * XOR of a 16-byte piece equals a fixed constant.  Timed over the same buffers
 * and launch sequence as a set of W4A16 calls, it measures what launching a
 * kernel and reading those bytes from cold memory costs at that size.
 *   src    device pointer, 16-byte aligned
 *   bytes  a multiple of 16 (0: no launch)
 *   sink   device uint32 (4-byte aligned), owned by the caller
 * Errors: INVALID_ARGUMENT (null src or sink with bytes > 0), INVALID_SHAPE
 * (bytes % 16), ALIGNMENT, HIP.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
