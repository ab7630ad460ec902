// Device scratch for the allocation-free forward (qlora_linear_fwd_noalloc):
// one file-scope array per GPU, of kScratchBytes, held by every GPU the
// library is loaded on until the process ends.  Its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and kept;
// host code uses only that address, never the array's name (which on the
// host is a stand-in symbol, not device memory).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace ql {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace ql
