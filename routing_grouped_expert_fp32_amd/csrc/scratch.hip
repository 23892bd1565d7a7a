// Workspace of the no-allocation entry point (beam_moe_forward_noalloc): one array per GPU, in
// device memory the library holds until the process ends.
#include <mutex>

#include "device_common.h"

// In host code `scratch` names a host-side stand-in, not the device array: the device address
// comes from hipGetSymbolAddress, once per device with that device current, and only that address
// is handed to kernels.
static __device__ __align__(256) unsigned char scratch[beam::kScratchBytes];

namespace beam {
namespace {
constexpr int kMaxDevices = 64;
}  // namespace

hipError_t scratch_of_current_device(void** out) {
  static void* ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace beam
