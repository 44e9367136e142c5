// Static device scratch of rpa_batch_attention_noalloc: the plan's metadata
// and the float32 partial outputs of split pieces, for callers that cannot
// allocate device memory.  One copy of the array exists on every GPU the
// library runs on, held until the process ends.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../launch.h"

// The array's name is a host-side stand-in on the host: kernels and copies
// take the device address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[rpa::kStaticScratchBytes];

namespace rpa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    // Once per device, with that device current.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace rpa
