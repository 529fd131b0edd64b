// Device-side scratch for the allocation-free forward (ha_attn_fwd_static).
//
// A file-scope device array of fixed size, kStaticScratchBytes, that every GPU the library
// runs on holds from the moment the code object is loaded there until the process ends. In
// host code its name is a host-side stand-in, not a device address: the address is looked
// up once per device (with that device current) through hipGetSymbolAddress and kept, and
// only that address is ever handed to kernels. Calls on one GPU share the array, which
// keeps the last call's contents; the forward writes every byte it reads before reading
// it, so nothing needs clearing between calls. Calls that overlap on one GPU race.
#include <mutex>

#include "ha_internal.h"

static __device__ __align__(256) char scratch[ha::kStaticScratchBytes];

namespace ha {
namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace ha
