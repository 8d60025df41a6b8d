// The fixed device scratch of the entry points that allocate nothing (cf_topk_select_noalloc):
// one file-scope device array per GPU, whose address is looked up once per device with that device
// current and kept. Host code never passes the array's name to a kernel: on the host that name is
// only a stand-in for the symbol, not a device address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cf.h"

static __device__ __align__(256) unsigned char scratch[CF_NOALLOC_SCRATCH_BYTES];

namespace cf {

constexpr int NOALLOC_MAX_DEVICES = 64;

// Device address of the scratch array on the current device (looked up on the first call per device).
hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[NOALLOC_MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace cf
