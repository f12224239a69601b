// Static device scratch of the entry point that allocates nothing
// (ra_ring_bwd_noalloc): the backward driver's fp32 delta workspace lives in a
// file-scope device array instead of caller memory.
//
// In host code the name `scratch` denotes a host-side stand-in, not device memory:
// passing it to a kernel would make the kernel fault.  Its device address is taken
// once per device, with that device current, by hipGetSymbolAddress, and only that
// address is ever handed to kernels.  Each GPU the library runs on holds its own copy
// of the array (at its own address) until the process ends.
#include <mutex>

#include "ra_internal.h"

static __device__ __align__(256) float scratch[ra::kStaticScratchBytes / sizeof(float)];

namespace ra {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ra
