// The library's own device scratch, for callers that cannot allocate: a
// file-scope device array that holds the split-K partials of mx_gemm_scratch
// in place of a caller workspace. Each GPU the library runs on keeps its own
// copy of the array, at its own address, until the process ends; the address
// is taken once per device (with that device current) by the first call on
// it and kept. The array's name is a host-side stand-in, never a device
// address: only the pointer returned by scratch_buffer reaches kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mx_launch.h"

namespace mx {

__attribute__((used)) static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_buffer(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace mx
