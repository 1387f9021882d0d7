// The decode's split-partial scratch as a static device array, for callers
// that cannot allocate device memory (code under graph capture, serving
// loops, harnesses that forbid hipMalloc).  Every GPU the library runs on
// holds its own copy of the array from the time the library's code object
// is loaded there until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address, so it is never passed to a kernel: the device address is looked up
// once per device with hipGetSymbolAddress (that device current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace pkv
