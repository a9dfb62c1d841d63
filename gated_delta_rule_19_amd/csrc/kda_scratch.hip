// The fixed device scratch of the allocation-free prefill entry point
// (kda_chunk_prefill_noalloc): a file-scope device array that every device
// the library runs on holds until the process ends.  Host code never passes
// the array's name to a kernel or a copy: its name is only a host-side
// stand-in.  The device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and cached here.
#include "kda_internal.h"

#include <mutex>

namespace kda {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
} // namespace

hipError_t noalloc_scratch(void **out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return e;
  if (dev < 0 || dev >= kMaxDevices)
    return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0)
      return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

} // namespace kda
