// Device scratch of mla_decode_fwd_noalloc: a file-scope device array that the
// code object holds on every GPU the library runs on (until the process
// ends), so that the entry point needs no allocation.  Host code never passes
// the array's name to a kernel or a copy: in host code that name is only a
// stand-in, not a device address.  The device address of this GPU's copy
// comes from hipGetSymbolAddress, looked up once per device with that device
// current, and is what the kernels receive.
#include "mla_internal.h"

#include <mutex>

namespace mla {
namespace {

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
