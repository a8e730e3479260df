// fa_scratch.hip -- the library's one fixed device array, which gives the
// entry point that allocates nothing (fa_bwd_noalloc) its workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` from the
// moment the code object is loaded on it until the process ends. In host
// code the name `scratch` is only a host-side stand-in, not a device
// address: host code uses the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {

static __device__ __align__(256) char scratch[FA_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
