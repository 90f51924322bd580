// Scratch memory of the no-allocation entry point (dspark_block_layer_noalloc).
//
// The scratch is one file-scope device array; each GPU the library runs on
// holds its own copy until the process ends. In host code the array's name
// is only a stand-in for the device symbol, so its device address is taken
// with hipGetSymbolAddress, once per device with that device current, and
// that address (never the name) is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace dspark {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dspark
