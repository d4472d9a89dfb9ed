// Static device scratch: the workspace of pkv_paged_decode_step_noalloc, for callers that
// cannot allocate device memory (code under graph capture, tight serving loops). Every
// device that loads the library holds its own copy of the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address; host code only
// ever uses the address hipGetSymbolAddress returns for the current device, kept per device.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_scratch.h"

static __device__ __align__(256) unsigned char scratch[pkv::kScratchBytes];

namespace pkv {

void* scratch_region() {
  static std::mutex mu;
  static void* addr[kScratchDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace pkv
