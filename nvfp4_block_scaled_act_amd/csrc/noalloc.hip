// Library-owned scratch memory for the allocation-free entry point
// (nvfp4_linear_noalloc): a file-scope device array, one copy per GPU, that
// holds the quantized activations of the dispatched linear's W4A4 route in
// place of a caller workspace.
//
// Host code never passes the array's name to a kernel or a copy: on the host
// that name is only a stand-in for the symbol, not a device address.  The
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; every use goes
// through it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/nvfp4.h"
#include "kernels.hpp"

namespace nvfp4 {

constexpr size_t kScratchBytes = NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES;  // per GPU, held until the process ends

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_pointer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace nvfp4
