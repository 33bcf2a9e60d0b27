// noalloc.hip -- the fixed scratch array behind selective_scan_fwd_noalloc.
//
// The scan's carries, hand-over flags and segment aggregates normally come from a
// stream-ordered pool.  Callers that must not allocate get them from this array instead:
// one copy per GPU, resident for the life of the process.  In host code the name `scratch`
// is only a stand-in for the symbol, not a device address; its address on the current
// device is looked up once per device with hipGetSymbolAddress and that pointer is what
// the kernels receive.  Calls on one GPU share the array, so calls that overlap in time on
// the same GPU (different streams, or host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssm_launch.h"

static __device__ __align__(256) unsigned char scratch[ssm::kNoAllocScratchBytes];

namespace ssm {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!q) return hipErrorInvalidSymbol;
    addr[dev] = q;
  }
  *ptr = addr[dev];
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

}  // namespace ssm
