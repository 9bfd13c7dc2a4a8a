// Static device scratch for the allocation-free entry points.
//
// One file-scope device array, sized once at build time, backs the scratch
// of sla_route_noalloc.  Every GPU the library runs on holds its own copy of
// the array (loaded with the code object) until the process ends.  The
// array's name is a host-side stand-in in host code, never a device
// address: the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that
// address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sla_internal.hpp"

namespace sla {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
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

}  // namespace sla
