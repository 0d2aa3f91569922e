// Device scratch for the allocation-free decode entry point
// (pkv_paged_attn_decode_noalloc): a file-scope device array that holds the
// split-context partial states the workspace argument holds otherwise.
//
// Host code must not pass the array's name to a kernel (on the host it is a
// stand-in, not a device address): the address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept.  Every call
// on a GPU shares that GPU's array; it keeps the last call's contents.
#include <mutex>

#include "kernels.h"

namespace pkv {

namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace pkv
