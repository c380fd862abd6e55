// The device-resident workspace of nsa_decode_fwd_noalloc: a fixed array that
// every GPU the library runs on holds until the process ends, for callers that
// cannot allocate (code under graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <atomic>

#include "nsa_internal.hpp"

namespace {

static __device__ __align__(256) char scratch[nsa::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
// Per device: the array's device address, taken once with that device current
// (in host code `scratch` names a host-side stand-in, not device memory).
std::atomic<void*> g_scratch_ptr[kMaxDevices];

}  // namespace

namespace nsa {

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // a racing first call stores the same address
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace nsa
