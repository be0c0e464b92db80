// Device scratch for the entry point that allocates nothing
// (tsel_colscore_noalloc): a file-scope array in the library's code object.
// The runtime places one copy of it on every GPU that loads the library, for
// the life of the process.  In host code the array's name is not a device
// address, so its address on the current device is looked up here, once per
// device, with hipGetSymbolAddress, and only that address is handed out.
#include <mutex>

#include "internal.h"

namespace tsel {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // scratch's address on each device, null until looked up

}  // namespace

hipError_t static_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace tsel
