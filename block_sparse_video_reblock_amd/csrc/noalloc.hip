// Device-resident scratch for the allocation-free entry point (bsa_summaries_noalloc).
//
// The array below lives in the library's code object: every GPU the library runs on holds one
// copy of it, at its own address, until the process ends.  Host code never passes the array's
// name to a kernel (on the host that name is only a stand-in for the symbol); it asks the
// runtime for the device address once per device, with that device current, and keeps it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[bsa::kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_init;

}  // namespace

namespace bsa {

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_init);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace bsa
