// Static device scratch of psa_estimate_mask_noalloc, the mask step for callers that
// cannot allocate device memory. One copy of the array per device, held until the
// process ends. Host code never uses `scratch` itself (on the host the name is only a
// stand-in for the symbol): each device's address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address reaches a kernel.
#include <mutex>

#include "psa.h"
#include "psa_launch.h"

static __device__ __align__(256) unsigned char scratch[PSA_NOALLOC_SCRATCH_BYTES];

namespace psa {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace psa
