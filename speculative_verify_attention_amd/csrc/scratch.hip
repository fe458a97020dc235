// scratch.hip - the fixed device scratch of spec_verify_attn_static: a
// file-scope device array that the library owns for the life of the
// process, so that a verify call needs no caller workspace and allocates
// nothing.
//
// In host code the array's name is only a host-side stand-in; its device
// address comes from hipGetSymbolAddress, resolved once per device with that
// device current, and that address is what kernels receive.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace svattn {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace svattn
