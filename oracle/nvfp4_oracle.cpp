// NVFP4 quantized linear -- CPU ORACLE.
//
// TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, obviously correct
// definition of what the GPU library computes.  Only the test suite, the smoke
// check and the CPU-baseline leg of the benchmark may load it.  It shares no
// source, header, table or helper with the GPU library, and the GPU library
// never loads it.
//
// What it follows (the pages):
//  * FlashInfer PR #3597 "Add BF16_FP4 GEMM ... for W4A16 workloads",
//    Description: the W4A16 product is (a @ dequant(b, b_sf).T) * alpha with
//    b_sf the per-16-element FP8-E4M3 block scales and alpha an fp32 scale.
//  * same page, API example: the weight global is (448 * 6) / max|w| and
//    alpha = 1 / g_w, handed to the kernel as an fp32 tensor.
//  * same page, review thread: an e2m1 nibble keeps its magnitude index in the
//    low three bits and its sign in bit 3.
//  * FreeToken PR #737, Changes: one row-major [N, K/2] code tensor with its
//    block scales serves both the W4A16 and the W4A4 linears, with one weight
//    global per tensor.
//  * FreeToken PR #736, Changes: the MoE gate_up GEMM applies the gated
//    activation and quantizes its output to NVFP4; the down GEMM applies the
//    routing weight and sums the top-k routes.
//
// Readings taken where the pages leave a step open (each is used below):
//  * scale and code decisions are made on the exact real values amax*g/6 and
//    |x|*g/S, by exact comparisons (no fp32 evaluation order is implied);
//  * both roundings are round-to-nearest, ties to the even code; values past
//    the largest finite value saturate (E4M3: 448, e2m1: 6);
//  * a block whose scale rounds to zero gets magnitude 0 in every code;
//  * a code keeps the sign bit of its input, so -0.0 and tiny negatives give 0x8;
//  * the element with even k sits in the low nibble of its byte;
//  * scales are stored row-major [rows, K/16], unswizzled;
//  * alpha is applied after the full-precision sum, before the bf16 rounding,
//    and the reference result is rounded once, from fp64, to bf16 (RNE);
//  * MoE: rows [0, I) of a gate_up expert are the gate, rows [I, 2I) the up
//    projection; h = SiLU(gate) * up, computed without a bf16 intermediate;
//    the top-k routes are summed at full precision and rounded once.
//
// Build: g++ -O2 -std=c++17 -fopenmp -shared -fPIC (no -ffast-math: the
// comparisons below rely on IEEE double arithmetic and a fused multiply-add).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Formats
// ---------------------------------------------------------------------------

// e2m1 (FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
// Exponent field 0 is subnormal: magnitude m/2.  Otherwise 2^(e-1) * (1 + m/2).
double e2m1_value(int code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

// OCP FP8 E4M3 ("E4M3FN"): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
// mantissa.  No infinities; exponent 15 with mantissa 7 is NaN.  Exponent 0 is
// subnormal: m * 2^-9.  Largest finite value 0x7E = 448.
double e4m3_value(int byte) {
  const int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  const double mag = (e == 0) ? std::ldexp(double(m), -9) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

double bf16_to_double(uint16_t bits) {
  uint32_t u = uint32_t(bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

double f32_to_double(float f) { return double(f); }

// bf16 = IEEE binary32 truncated to its top 16 bits: 8 significant bits,
// exponent range of fp32.  Round a double to the nearest bf16, ties to even.
uint16_t bf16_rne(double r) {
  if (std::isnan(r)) return 0x7FC0;
  const uint16_t sign = std::signbit(r) ? 0x8000 : 0;
  const double a = std::fabs(r);
  if (a == 0.0) return sign;
  int ex;
  std::frexp(a, &ex);                          // a = f * 2^ex, f in [0.5, 1)
  const int lead = ex - 1;                     // exponent of the leading bit
  const int quantum = (lead < -126 ? -126 : lead) - 7;  // 7 stored mantissa bits
  const double n = std::nearbyint(std::ldexp(a, -quantum));  // default mode: ties to even
  const double v = std::ldexp(n, quantum);
  const double max_bf16 = std::ldexp(255.0, 127 - 7);        // 0x7F7F
  if (v > max_bf16) return uint16_t(sign | 0x7F80);          // overflow -> inf
  const float fv = float(v);                                 // exact
  uint32_t u;
  std::memcpy(&u, &fv, 4);
  return uint16_t(sign | (u >> 16));
}

// The finite non-negative values of a format in increasing order; the index
// is the code (e2m1 magnitude index 0..7, E4M3 byte 0x00..0x7E).
struct Grid {
  std::vector<double> v;
};

Grid make_e2m1_grid() {
  Grid g;
  for (int c = 0; c < 8; ++c) g.v.push_back(e2m1_value(c));
  return g;
}

Grid make_e4m3_grid() {
  Grid g;
  for (int b = 0; b <= 0x7E; ++b) g.v.push_back(e4m3_value(b));
  return g;
}

const Grid& E2M1() {
  static const Grid g = make_e2m1_grid();
  return g;
}
const Grid& E4M3() {
  static const Grid g = make_e4m3_grid();
  return g;
}

// Sign of (x * y - t), computed exactly: the fused multiply-add forms x*y - t
// without intermediate rounding and its single rounding keeps the sign (the
// operands here are far from the subnormal range, where it could not).
int sign_of_product_minus(double x, double y, double t) {
  const double d = std::fma(x, y, -t);
  return (d > 0) - (d < 0);
}

// Round the exact real value x*y/den to the nearest grid value, ties to the
// even index, values past the last grid point saturating to it.  x*y is never
// formed in floating point: it is compared against den * midpoint, which is
// exact in double (den has at most 4 significant bits, midpoints at most 5).
int round_to_grid(double x, double y, double den, const Grid& grid) {
  const std::vector<double>& v = grid.v;
  const int n = int(v.size());
  // lo = the largest index with v[lo] <= x*y/den (v[0] = 0 <= any magnitude).
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (sign_of_product_minus(x, y, den * v[mid]) >= 0) lo = mid; else hi = mid - 1;
  }
  if (lo == n - 1) return lo;  // at or beyond the largest value: saturate
  const double midpoint = den * 0.5 * (v[lo] + v[lo + 1]);
  const int c = sign_of_product_minus(x, y, midpoint);
  if (c < 0) return lo;
  if (c > 0) return lo + 1;
  return (lo % 2 == 0) ? lo : lo + 1;  // exact tie: the even index
}

// Distance, relative to the value, from x*y/den to the nearest rounding
// boundary (grid midpoint) -- a diagnostic used to tell a benign code flip
// (a result straddling a boundary by a rounding error) from a wrong code.
double boundary_margin(double x, double y, double den, const Grid& grid) {
  const double val = x * y / den;  // approximate, only for the diagnostic
  double best = std::numeric_limits<double>::infinity();
  for (size_t i = 0; i + 1 < grid.v.size(); ++i) {
    const double midpoint = 0.5 * (grid.v[i] + grid.v[i + 1]);
    const double d = std::fabs(val - midpoint) / (midpoint > 0 ? midpoint : 1.0);
    if (d < best) best = d;
  }
  return best;
}

// ---------------------------------------------------------------------------
// NVFP4 quantization of one 16-element block under a global scale g.
//   amax  = max |x_i|
//   s     = E4M3 byte nearest to amax*g/6 (saturating at 448)
//   S     = value of s
//   c_i   = sign(x_i) << 3 | e2m1 index nearest to |x_i|*g/S (saturating at 6)
// ---------------------------------------------------------------------------
struct Block {
  uint8_t scale;
  uint8_t code[16];
};

Block quantize_block(const double* x, double g) {
  Block b;
  double amax = 0.0;
  for (int i = 0; i < 16; ++i) amax = std::fmax(amax, std::fabs(x[i]));
  b.scale = uint8_t(round_to_grid(amax, g, 6.0, E4M3()));
  const double S = e4m3_value(b.scale);
  for (int i = 0; i < 16; ++i) {
    const int sign = std::signbit(x[i]) ? 1 : 0;
    const int mag = (S == 0.0) ? 0 : round_to_grid(std::fabs(x[i]), g, S, E2M1());
    b.code[i] = uint8_t(sign << 3 | mag);
  }
  return b;
}

void store_block(const Block& b, uint8_t* code_row, uint8_t* scale_row, int64_t j) {
  scale_row[j] = b.scale;
  for (int i = 0; i < 8; ++i)
    code_row[8 * j + i] = uint8_t(b.code[2 * i] | (b.code[2 * i + 1] << 4));
}

// Dequantized value of element k of a row: e2m1(code) * E4M3(scale of k/16).
double dequant(const uint8_t* code_row, const uint8_t* scale_row, int64_t k) {
  const uint8_t byte = code_row[k / 2];
  const int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
  return e2m1_value(code) * e4m3_value(scale_row[k / 16]);
}

// The same value as an integer in units of 2^-10 (e2m1 values are multiples of
// 1/2 and E4M3 values multiples of 2^-9): |value| <= 6*448*2^10 < 2^22.
int64_t dequant_units(const uint8_t* code_row, const uint8_t* scale_row, int64_t k) {
  const double v = dequant(code_row, scale_row, k) * 1024.0;  // exact
  return int64_t(v);
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

}  // namespace

// ---------------------------------------------------------------------------
// C ABI (loaded through ctypes by the tests).
// ---------------------------------------------------------------------------
extern "C" {

double orc_e2m1_value(int code) { return e2m1_value(code & 15); }
double orc_e4m3_value(int byte) { return e4m3_value(byte & 255); }

// Nearest E4M3 byte (0x00..0x7E) to the exact value x*y/den; RNE, saturating.
int orc_e4m3_round(double x, double y, double den) { return round_to_grid(x, y, den, E4M3()); }
// Nearest e2m1 magnitude index (0..7) to the exact value x*y/den; RNE, saturating.
int orc_e2m1_round(double x, double y, double den) { return round_to_grid(x, y, den, E2M1()); }

uint16_t orc_bf16_rne(double r) { return bf16_rne(r); }

// Global scale of a bf16 tensor: fp32(448 * 6 / max|x|), the quotient rounded
// once to fp32 as an fp32 division would (a double quotient of two fp32 values
// rounds to the same fp32).  Returns 0 for an all-zero tensor.
float orc_global_scale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
  double amax = 0.0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) amax = std::fmax(amax, std::fabs(bf16_to_double(x[r * ld + c])));
  if (amax == 0.0) return 0.0f;
  return float(2688.0 / amax);
}

// Global scale from an already-known amax (a double): fp32(2688 / amax).
float orc_global_scale_from_amax(double amax) { return amax > 0 ? float(2688.0 / amax) : 0.0f; }

// alpha = fp32(1 / (g_w * g_a)), the product and the quotient taken in double
// as the pages' Python does; g_a <= 0 means "no activation global" (W4A16).
float orc_alpha(float g_w, float g_a) {
  const double den = (g_a > 0.0f) ? double(g_w) * double(g_a) : double(g_w);
  return float(1.0 / den);
}

// Quantize bf16 rows [rows, K] (row stride ld elements) under the global g.
// codes: [rows, K/2] row-major; scales: [rows, K/16] row-major.  K % 16 == 0.
void orc_quantize_bf16(const uint16_t* x, int64_t rows, int64_t K, int64_t ld, float g,
                       uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[16];
    for (int64_t j = 0; j < K / 16; ++j) {
      for (int i = 0; i < 16; ++i) blk[i] = bf16_to_double(x[r * ld + 16 * j + i]);
      store_block(quantize_block(blk, double(g)), codes + r * (K / 2), scales + r * (K / 16), j);
    }
  }
}

// Same for fp64 inputs (the MoE's h, which is never rounded to bf16).
void orc_quantize_f64(const double* x, int64_t rows, int64_t K, int64_t ld, float g,
                      uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < K / 16; ++j)
      store_block(quantize_block(x + r * ld + 16 * j, double(g)), codes + r * (K / 2),
                  scales + r * (K / 16), j);
}

// Dequantize [rows, K] NVFP4 to fp64 (exact).
void orc_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) out[r * K + k] = dequant(codes + r * (K / 2), scales + r * (K / 16), k);
}

// W4A16 linear on selected outputs:
//   ref[i, j] = alpha * sum_k a[rows[i], k] * dequant(W)[cols[j], k]   (fp64)
//   out[i, j] = bf16_rne(ref[i, j]);  sabs[i, j] = alpha * sum_k |a * w|
// rows/cols may be null (all M rows / all N columns).  Outputs are dense
// [n_rows, n_cols].  a: bf16 [M, K] with row stride lda.
void orc_linear_w4a16(const uint16_t* a, int64_t lda, const int64_t* rows, int64_t n_rows,
                      const uint8_t* w_codes, const uint8_t* w_scales, int64_t K,
                      const int64_t* cols, int64_t n_cols, float alpha,
                      uint16_t* out, double* ref, double* sabs) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t jj = 0; jj < n_cols; ++jj) {
    const int64_t n = cols ? cols[jj] : jj;
    std::vector<double> w(K);
    for (int64_t k = 0; k < K; ++k) w[k] = dequant(w_codes + n * (K / 2), w_scales + n * (K / 16), k);
    for (int64_t ii = 0; ii < n_rows; ++ii) {
      const int64_t m = rows ? rows[ii] : ii;
      double acc = 0.0, acc_abs = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double p = bf16_to_double(a[m * lda + k]) * w[k];  // exact product
        acc += p;
        acc_abs += std::fabs(p);
      }
      const double r = double(alpha) * acc;
      if (ref) ref[ii * n_cols + jj] = r;
      if (sabs) sabs[ii * n_cols + jj] = double(alpha) * acc_abs;
      if (out) out[ii * n_cols + jj] = bf16_rne(r);
    }
  }
}

// W4A4 linear on selected outputs, with an exact integer dot product:
// dequantized values are integers in units of 2^-10, products in units of
// 2^-20 (< 2^44), and a sum over K < 2^13 terms stays below 2^57.
//   ref = alpha * sum * 2^-20 (fp64), out = bf16_rne(ref).
void orc_linear_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const int64_t* rows, int64_t n_rows,
                     const uint8_t* w_codes, const uint8_t* w_scales, int64_t K,
                     const int64_t* cols, int64_t n_cols, float alpha,
                     uint16_t* out, double* ref, double* sabs) {
  // Dequantize the selected A rows once.
  std::vector<int64_t> A(size_t(n_rows) * K);
#pragma omp parallel for schedule(static)
  for (int64_t ii = 0; ii < n_rows; ++ii) {
    const int64_t m = rows ? rows[ii] : ii;
    for (int64_t k = 0; k < K; ++k) A[ii * K + k] = dequant_units(a_codes + m * (K / 2), a_scales + m * (K / 16), k);
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t jj = 0; jj < n_cols; ++jj) {
    const int64_t n = cols ? cols[jj] : jj;
    std::vector<int64_t> w(K);
    for (int64_t k = 0; k < K; ++k) w[k] = dequant_units(w_codes + n * (K / 2), w_scales + n * (K / 16), k);
    for (int64_t ii = 0; ii < n_rows; ++ii) {
      int64_t acc = 0, acc_abs = 0;
      const int64_t* ar = &A[ii * K];
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = ar[k] * w[k];
        acc += p;
        acc_abs += p < 0 ? -p : p;
      }
      const double r = double(alpha) * std::ldexp(double(acc), -20);
      if (ref) ref[ii * n_cols + jj] = r;
      if (sabs) sabs[ii * n_cols + jj] = double(alpha) * std::ldexp(double(acc_abs), -20);
      if (out) out[ii * n_cols + jj] = bf16_rne(r);
    }
  }
}

}  // extern "C"

namespace {

// The pairs q = tt*top_k + r of the selected tokens (tt indexes `tokens`, or
// is the token itself when `tokens` is null) routed to each expert, in pair
// order.  A pair whose id lies outside [0, E) belongs to no expert: it is
// skipped and adds nothing to its token's sum.
std::vector<std::vector<int64_t>> pairs_by_expert(const int32_t* ids, const int64_t* tokens, int64_t n_tok,
                                                  int64_t top_k, int64_t E) {
  std::vector<std::vector<int64_t>> by(static_cast<size_t>(E));
  for (int64_t tt = 0; tt < n_tok; ++tt) {
    const int64_t t = tokens ? tokens[tt] : tt;
    for (int64_t r = 0; r < top_k; ++r) {
      const int64_t e = ids[t * top_k + r];
      if (e >= 0 && e < E) by[size_t(e)].push_back(tt * top_k + r);
    }
  }
  return by;
}

}  // namespace

extern "C" {

// NVFP4 MoE expert layer (W4A4 on both GEMMs) for selected tokens.
//   x      : bf16 [T, K] hidden states
//   ids, w : [T, top_k] expert ids (int32) and routing weights (fp32)
//   gate_up: codes [E, 2I, K/2], scales [E, 2I, K/16]
//   down   : codes [E, K, I/2], scales [E, K, I/16]
//   g1, g2 : static activation globals of the two GEMM inputs
//   alpha_gu[e] = fp32(1/(g_gu[e]*g1)), alpha_dn[e] = fp32(1/(g_dn[e]*g2))
// For each selected token t and route r whose expert id e lies in [0, E)
// (a route with any other id is skipped and adds nothing):
//   z[j]   = alpha_gu[e] * <dequant(q(x_t; g1)), dequant(gate_up[e])[j]>, j < 2I (exact sum)
//   h[i]   = SiLU(z[i]) * z[I + i]                                 (fp64, i < I)
//   y[k]   = alpha_dn[e] * <dequant(q(h; g2)), dequant(down[e])[k]> (exact sum)
//   out[t] = bf16_rne(sum_r w[t, r] * y_r)       (fp64, routes added in order r = 0, 1, ...)
// The work runs expert by expert, each expert's banks dequantized once; the
// sums and their order are the ones written above.
// Per (token, route) the oracle's own h codes/scales are returned
// ([n_tok*top_k, I/2], [n_tok*top_k, I/16]; zeros for a skipped pair) with,
// per h element, the relative distance of |h|*g2/S to the nearest e2m1
// rounding boundary, and per h block the relative distance of amax*g2/6 to
// the nearest E4M3 boundary (margins tell a benign rounding flip from a
// wrong code; infinite for a skipped pair).  ref/sabs as for the linears.
// h_amax (optional, one double) receives max |h| over the computed pairs.
void orc_moe_w4a4(const uint16_t* x, int64_t T, int64_t K, const int32_t* ids, const float* rw,
                  int64_t top_k, int64_t E, int64_t I,
                  const uint8_t* gu_codes, const uint8_t* gu_scales,
                  const uint8_t* dn_codes, const uint8_t* dn_scales,
                  float g1, float g2, const float* alpha_gu, const float* alpha_dn,
                  const int64_t* tokens, int64_t n_tok,
                  uint8_t* h_codes, uint8_t* h_scales, double* h_code_margin, double* h_scale_margin,
                  double* h_amax, uint16_t* out, double* ref, double* sabs) {
  (void)T;
  const int64_t twoI = 2 * I, P = n_tok * top_k;
  const double inf = std::numeric_limits<double>::infinity();

  // Each selected token's hidden state quantized under g1, dequantized in 2^-10 units.
  std::vector<int64_t> xa(size_t(n_tok * K));
#pragma omp parallel for schedule(static)
  for (int64_t tt = 0; tt < n_tok; ++tt) {
    const int64_t t = tokens ? tokens[tt] : tt;
    std::vector<uint8_t> xc(K / 2), xs(K / 16);
    orc_quantize_bf16(x + t * K, 1, K, K, g1, xc.data(), xs.data());
    for (int64_t k = 0; k < K; ++k) xa[size_t(tt * K + k)] = dequant_units(xc.data(), xs.data(), k);
  }

  // Skipped pairs: no h, infinite margins, nothing added.
  for (int64_t p = 0; p < P; ++p) {
    std::memset(h_codes + p * (I / 2), 0, size_t(I / 2));
    std::memset(h_scales + p * (I / 16), 0, size_t(I / 16));
    if (h_code_margin)
      for (int64_t i = 0; i < I; ++i) h_code_margin[p * I + i] = inf;
    if (h_scale_margin)
      for (int64_t b = 0; b < I / 16; ++b) h_scale_margin[p * (I / 16) + b] = inf;
  }

  // y[p] = alpha_dn * exact down sum of pair p, ya[p] = the same of |products|.
  std::vector<double> y(size_t(P * K), 0.0), ya(size_t(P * K), 0.0);
  const std::vector<std::vector<int64_t>> by_expert = pairs_by_expert(ids, tokens, n_tok, top_k, E);
  std::vector<int64_t> wgu, wdn;
  double amax_all = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    const std::vector<int64_t>& pe = by_expert[size_t(e)];
    if (pe.empty()) continue;
    // The expert's two banks, dequantized once (2^-10 units).
    const uint8_t* guc = gu_codes + e * twoI * (K / 2);
    const uint8_t* gus = gu_scales + e * twoI * (K / 16);
    const uint8_t* dnc = dn_codes + e * K * (I / 2);
    const uint8_t* dns = dn_scales + e * K * (I / 16);
    wgu.resize(size_t(twoI * K));
    wdn.resize(size_t(K * I));
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < twoI; ++j)
      for (int64_t k = 0; k < K; ++k) wgu[size_t(j * K + k)] = dequant_units(guc + j * (K / 2), gus + j * (K / 16), k);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
      for (int64_t i = 0; i < I; ++i) wdn[size_t(k * I + i)] = dequant_units(dnc + k * (I / 2), dns + k * (I / 16), i);

#pragma omp parallel for schedule(dynamic, 1) reduction(max : amax_all)
    for (size_t q = 0; q < pe.size(); ++q) {
      const int64_t p = pe[q], tt = p / top_k;
      const int64_t* xr = &xa[size_t(tt * K)];
      // gate_up, then the gated activation in fp64
      std::vector<double> z(twoI);
      for (int64_t j = 0; j < twoI; ++j) {
        const int64_t* wr = &wgu[size_t(j * K)];
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += xr[k] * wr[k];
        z[j] = double(alpha_gu[e]) * std::ldexp(double(s), -20);
      }
      std::vector<double> h(I);
      for (int64_t i = 0; i < I; ++i) {
        h[i] = silu(z[i]) * z[I + i];
        amax_all = std::fmax(amax_all, std::fabs(h[i]));
      }
      // h quantized under g2, with its boundary margins
      uint8_t* hc = h_codes + p * (I / 2);
      uint8_t* hs = h_scales + p * (I / 16);
      orc_quantize_f64(h.data(), 1, I, I, g2, hc, hs);
      for (int64_t b = 0; b < I / 16; ++b) {
        const double S = e4m3_value(hs[b]);
        double bmax = 0.0;
        for (int i = 0; i < 16; ++i) bmax = std::fmax(bmax, std::fabs(h[16 * b + i]));
        if (h_scale_margin) h_scale_margin[p * (I / 16) + b] = boundary_margin(bmax, double(g2), 6.0, E4M3());
        for (int i = 0; i < 16; ++i) {
          const int64_t idx = 16 * b + i;
          if (h_code_margin)
            h_code_margin[p * I + idx] =
                (S == 0.0) ? inf : boundary_margin(std::fabs(h[idx]), double(g2), S, E2M1());
        }
      }
      // down on the quantized h
      std::vector<int64_t> ha(I);
      for (int64_t i = 0; i < I; ++i) ha[i] = dequant_units(hc, hs, i);
      for (int64_t k = 0; k < K; ++k) {
        const int64_t* wr = &wdn[size_t(k * I)];
        int64_t s = 0, sa = 0;
        for (int64_t i = 0; i < I; ++i) {
          const int64_t prod = ha[i] * wr[i];
          s += prod;
          sa += prod < 0 ? -prod : prod;
        }
        y[size_t(p * K + k)] = double(alpha_dn[e]) * std::ldexp(double(s), -20);
        ya[size_t(p * K + k)] = double(alpha_dn[e]) * std::ldexp(double(sa), -20);
      }
    }
  }

  // Each token's routes, added in order r = 0, 1, ... and rounded once.
#pragma omp parallel for schedule(static)
  for (int64_t tt = 0; tt < n_tok; ++tt) {
    const int64_t t = tokens ? tokens[tt] : tt;
    std::vector<double> acc(K, 0.0), acc_abs(K, 0.0);
    for (int64_t r = 0; r < top_k; ++r) {
      const int64_t e = ids[t * top_k + r];
      if (e < 0 || e >= E) continue;
      const int64_t p = tt * top_k + r;
      const double wr = double(rw[t * top_k + r]);
      for (int64_t k = 0; k < K; ++k) {
        acc[k] += wr * y[size_t(p * K + k)];
        acc_abs[k] += std::fabs(wr) * ya[size_t(p * K + k)];
      }
    }
    for (int64_t k = 0; k < K; ++k) {
      if (ref) ref[tt * K + k] = acc[k];
      if (sabs) sabs[tt * K + k] = acc_abs[k];
      if (out) out[tt * K + k] = bf16_rne(acc[k]);
    }
  }
  if (h_amax) *h_amax = amax_all;
}

// NVFP4 MoE expert layer with W4A16 on both GEMMs (bf16 x and h), for
// selected tokens; banks and ids/w as orc_moe_w4a4, alpha_gu[e] =
// fp32(1/g_gu[e]), alpha_dn[e] = fp32(1/g_dn[e]).  For each selected token t
// and route r whose id e lies in [0, E) (other ids are skipped):
//   z[j]   = alpha_gu[e] * sum_k x[t, k] * dequant(gate_up[e])[j, k]   (fp64)
//   h[i]   = SiLU(z[i]) * z[I + i]                                     (fp64)
//   hb[i]  = bf16_rne(h[i]), or h_in[pair][i] when h_in is given
//   y[n]   = alpha_dn[e] * sum_i hb[i] * dequant(down[e])[n, i]        (fp64)
//   out[t] = bf16_rne(sum_r w[t, r] * y_r)       (fp64, routes added in order r = 0, 1, ...)
// The work runs expert by expert, each expert's banks dequantized once.
// Per pair q = tt*top_k + r (tt: index into tokens): h_bits[q] = bf16_rne(h),
// h_ref[q] = h, and h_sabs[q] = |SiLU'(z_g)| |z_u| Sg + |SiLU(z_g)| Su, Sg
// and Su being alpha_gu * sum |x w| of the two dot products (the scale of h's
// error from fp32 sums); zeros for a skipped pair.  ref/sabs as the linears.
void orc_moe_w4a16(const uint16_t* x, int64_t T, int64_t K, const int32_t* ids, const float* rw,
                   int64_t top_k, int64_t E, int64_t I,
                   const uint8_t* gu_codes, const uint8_t* gu_scales,
                   const uint8_t* dn_codes, const uint8_t* dn_scales,
                   const float* alpha_gu, const float* alpha_dn, const int64_t* tokens, int64_t n_tok,
                   const uint16_t* h_in, uint16_t* h_bits, double* h_ref, double* h_sabs,
                   uint16_t* out, double* ref, double* sabs) {
  (void)T;
  const int64_t twoI = 2 * I, P = n_tok * top_k;
  for (int64_t q = 0; q < P * I; ++q) {  // skipped pairs keep these zeros
    if (h_bits) h_bits[q] = 0;
    if (h_ref) h_ref[q] = 0.0;
    if (h_sabs) h_sabs[q] = 0.0;
  }
  // s[p] = the down sum of pair p, sa[p] = the same of |products|.
  std::vector<double> ys(size_t(P * K), 0.0), ysa(size_t(P * K), 0.0);
  const std::vector<std::vector<int64_t>> by_expert = pairs_by_expert(ids, tokens, n_tok, top_k, E);
  std::vector<double> wgu, wdn;
  for (int64_t e = 0; e < E; ++e) {
    const std::vector<int64_t>& pe = by_expert[size_t(e)];
    if (pe.empty()) continue;
    // The expert's two banks, dequantized once (exact in fp64).
    const uint8_t* guc = gu_codes + e * twoI * (K / 2);
    const uint8_t* gus = gu_scales + e * twoI * (K / 16);
    const uint8_t* dnc = dn_codes + e * K * (I / 2);
    const uint8_t* dns = dn_scales + e * K * (I / 16);
    wgu.resize(size_t(twoI * K));
    wdn.resize(size_t(K * I));
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < twoI; ++j)
      for (int64_t k = 0; k < K; ++k) wgu[size_t(j * K + k)] = dequant(guc + j * (K / 2), gus + j * (K / 16), k);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < K; ++n)
      for (int64_t i = 0; i < I; ++i) wdn[size_t(n * I + i)] = dequant(dnc + n * (I / 2), dns + n * (I / 16), i);

#pragma omp parallel for schedule(dynamic, 1)
    for (size_t qq = 0; qq < pe.size(); ++qq) {
      const int64_t q = pe[qq], tt = q / top_k;
      const int64_t t = tokens ? tokens[tt] : tt;
      std::vector<double> xv(K);
      for (int64_t k = 0; k < K; ++k) xv[k] = bf16_to_double(x[t * K + k]);
      std::vector<double> z(twoI), za(twoI);
      for (int64_t j = 0; j < twoI; ++j) {
        const double* wr = &wgu[size_t(j * K)];
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double p = xv[k] * wr[k];  // exact product
          s += p;
          sa += std::fabs(p);
        }
        z[j] = double(alpha_gu[e]) * s;
        za[j] = double(alpha_gu[e]) * sa;
      }
      std::vector<double> hb(I);
      for (int64_t i = 0; i < I; ++i) {
        const double zg = z[i], zu = z[I + i];
        const double sig = 1.0 / (1.0 + std::exp(-zg));
        const double h = silu(zg) * zu;
        const double dsilu = sig + zg * sig * (1.0 - sig);
        const uint16_t bits = bf16_rne(h);
        if (h_bits) h_bits[q * I + i] = bits;
        if (h_ref) h_ref[q * I + i] = h;
        if (h_sabs) h_sabs[q * I + i] = std::fabs(dsilu) * std::fabs(zu) * za[i] + std::fabs(silu(zg)) * za[I + i];
        hb[i] = bf16_to_double(h_in ? h_in[q * I + i] : bits);
      }
      for (int64_t n = 0; n < K; ++n) {
        const double* wr = &wdn[size_t(n * I)];
        double s = 0.0, sa = 0.0;
        for (int64_t i = 0; i < I; ++i) {
          const double p = hb[i] * wr[i];  // exact product
          s += p;
          sa += std::fabs(p);
        }
        ys[size_t(q * K + n)] = s;
        ysa[size_t(q * K + n)] = sa;
      }
    }
  }

  // Each token's routes, added in order r = 0, 1, ... and rounded once.
#pragma omp parallel for schedule(static)
  for (int64_t tt = 0; tt < n_tok; ++tt) {
    const int64_t t = tokens ? tokens[tt] : tt;
    std::vector<double> acc(K, 0.0), acc_abs(K, 0.0);
    for (int64_t r = 0; r < top_k; ++r) {
      const int64_t e = ids[t * top_k + r];
      if (e < 0 || e >= E) continue;
      const int64_t q = tt * top_k + r;
      const double wr = double(rw[t * top_k + r]);
      for (int64_t n = 0; n < K; ++n) {
        acc[n] += wr * (double(alpha_dn[e]) * ys[size_t(q * K + n)]);
        acc_abs[n] += std::fabs(wr) * double(alpha_dn[e]) * ysa[size_t(q * K + n)];
      }
    }
    for (int64_t n = 0; n < K; ++n) {
      if (ref) ref[tt * K + n] = acc[n];
      if (sabs) sabs[tt * K + n] = acc_abs[n];
      if (out) out[tt * K + n] = bf16_rne(acc[n]);
    }
  }
}

}  // extern "C"
