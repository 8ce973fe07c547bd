// Device scratch for the entry point that allocates nothing
// (moba_forward_noalloc): one file-scope array per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns, taken once per device with that device
// current and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace moba {

static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxGridCacheDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxGridCacheDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return e != hipSuccess ? e : hipErrorInvalidSymbol;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moba
