// Streaming-read diagnostic: reads a buffer once, one 16-byte nontemporal
// load per thread (the largest per-lane load, every wave covering whole cache
// lines), the way the W4A16 kernels read their weight units, and computes
// nothing from the data beyond an XOR that is stored only in the rare case it
// equals a fixed constant (so the loads cannot be dropped).  Timed over the
// same buffers and launch sequence as a set of linear calls, it gives the
// time a kernel needs just to launch and read those bytes from cold memory.
#include "device.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 v = ld16_nt(src + 16 * i);
  const uint32_t x = v.x ^ v.y ^ v.z ^ v.w;
  if (x == 0x6a09e667u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(stream_read_kernel, dim3(uint32_t(blocks)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
