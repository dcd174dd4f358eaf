// The library's static device scratch: the workspace of the entry point that
// allocates nothing (fce_fused_fwd_bwd_noalloc), for callers that cannot
// allocate device memory.
//
// `scratch` is a file-scope device array of kStaticScratchBytes.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a host-side stand-in, never a device
// address: the first call on a device looks up that device's copy with
// hipGetSymbolAddress (with the device current) and keeps the address per
// device; kernels get that address, as they get a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fce.h"
#include "fce_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FCE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {nullptr};

}  // namespace

namespace fce {

hipError_t static_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  *bytes = FCE_STATIC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace fce
