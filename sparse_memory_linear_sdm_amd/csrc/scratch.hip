// The library's own device scratch buffer, for the entry points that must not
// allocate (sdm_scan_backward_noalloc): a file-scope device array that every
// GPU the library runs on holds from the module load until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address on the current GPU is looked up once per device with
// hipGetSymbolAddress and cached; every host use of the buffer (kernel
// arguments) goes through that address.  All calls on one GPU share its copy.
#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[sdm::kStaticScratchBytes];

namespace sdm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sdm
