// Scratch memory of the allocation-free routing entry point.
//
// Callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) call moe_init_routing_noalloc,
// whose scratch (the routing histograms and, for a gather-type index, the scatter
// index) lives in the file-scope array below instead of a caller workspace. Each GPU
// holds its own copy of the array from the library's load until the process ends; its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept. Host code never passes the array's name to a kernel: on the host
// that name is only a stand-in for the symbol, not a device address.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
