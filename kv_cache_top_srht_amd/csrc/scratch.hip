// Library-owned device scratch for the retrieval entry point that allocates
// nothing (pariskv_retrieve_topk_noalloc): one file-scope device array per
// GPU, loaded with the library's code object and held until the process
// ends.  Host code never passes the array's name to a kernel (on the host
// that name is only a stand-in, not a device address); it passes the address
// hipGetSymbolAddress returns for the current device, resolved once per
// device on the first call there and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pariskv_internal.h"

namespace pkv {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace pkv
