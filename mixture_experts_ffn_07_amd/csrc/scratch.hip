// Library-owned device scratch for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): moe_decode_forward_noalloc keeps its workspace here instead of
// in a caller-supplied buffer.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// must not pass the array's name to a kernel (on the host it names a stand-in,
// not device memory); static_scratch() returns the device address that
// hipGetSymbolAddress reports for the current device, taken once per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
