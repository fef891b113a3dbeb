// One-time re-tiling of an NVFP4 weight into the MFMA-native tiled layout read
// by both linears (FlashInfer PR #3597, API: a prepare step run once per weight
// so the GEMM can dequantize fast; FreeToken PR #737, Changes: both linears use
// one weight copy).
//
// Input: the checkpoint's row-major codes [N, K/2] (two e2m1 per byte, even k
// in the low nibble) and E4M3 scales [N, K/16].
//
// Output: ceil(N/16) * (K/256) units of 2304 bytes, unit (t, s) at
// (t * K/256 + s) * 2304, covering rows 16t..16t+15 and k in [256s, 256s+256).
// Inside a unit the 64 "lanes" l = r + 16q (r = row in the tile, q = 0..3) own
// the four 16-k scale groups g = 4p + q (p = 0..3) of their row:
//   bytes [16l, 16l+16)           codes of groups q and 4+q   (8 bytes each)
//   bytes [1024+16l, 1024+16l+16) codes of groups 8+q and 12+q
//   bytes [2048+4l, 2048+4l+4)    scale bytes of groups q, 4+q, 8+q, 12+q
// so one wave reads a unit as three fully coalesced loads (two dwordx4, one
// dword per lane) and every lane holds exactly the operand of its 16x16x32
// MFMA row.  Rows >= N are zero (code 0, scale 0).
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(256) void retile_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                     int32_t N, int32_t K, int64_t units, uint8_t* __restrict__ dst,
                                                     int32_t swz_cols) {
  const int64_t gid = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // one wave per unit
  if (gid >= units) return;
  const int lane = int(threadIdx.x & 63);
  const int r = lane & 15, q = lane >> 4;
  const int32_t steps = K / 256;
  const int64_t t = gid / steps, s = gid - t * steps;
  const int64_t row = t * 16 + r;
  uint2 c[4] = {make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0)};
  uint32_t sc = 0;
  if (row < N) {
    const uint8_t* crow = codes + row * (K / 2) + s * 128;
    const uint8_t* srow = scales + row * (K / 16) + s * 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      c[p] = *reinterpret_cast<const uint2*>(crow + 32 * p + 8 * q);
      const uint8_t sb = swz_cols > 0 ? scales[swizzled_scale_offset(row, s * 16 + 4 * p + q, swz_cols)]
                                      : srow[4 * p + q];
      sc |= uint32_t(sb) << (8 * p);
    }
  }
  uint8_t* u = dst + gid * 2304;
  *reinterpret_cast<uint4*>(u + 16 * lane) = make_uint4(c[0].x, c[0].y, c[1].x, c[1].y);
  *reinterpret_cast<uint4*>(u + 1024 + 16 * lane) = make_uint4(c[2].x, c[2].y, c[3].x, c[3].y);
  *reinterpret_cast<uint32_t*>(u + 2048 + 4 * lane) = sc;
}

}  // namespace

int64_t tiled_weight_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * (K / 256) * 2304; }

hipError_t launch_retile(const void* codes, const void* scales, int64_t N, int64_t K, void* dst, hipStream_t stream,
                         int64_t swz_cols) {
  const int64_t units = (N + 15) / 16 * (K / 256);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(retile_kernel, dim3(uint32_t((units + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales), int32_t(N), int32_t(K),
                     units, static_cast<uint8_t*>(dst), int32_t(swz_cols));
  return hipGetLastError();
}

}  // namespace nvfp4
