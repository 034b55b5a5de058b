// Fixed device scratch for the call that allocates nothing
// (ff_render_attend_static_scratch): the split-item partials of one renderer
// call live in this file-scope array instead of the caller's workspace.
//
// Every device the library runs on holds its own copy of the array (at its
// own address) until the process ends.  Host code never passes the array's
// name to a kernel: its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../ff_internal.h"

namespace ff {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

int dev_static_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* ptr_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FF_E_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr_of[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FF_E_HIP;
    ptr_of[dev] = p;
  }
  *ptr = ptr_of[dev];
  *bytes = kStaticScratchBytes;
  return 0;
}

}  // namespace ff
