// The workspace of dsa_forward_noalloc: a device array the library owns, so
// that callers who cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc) can still
// run the whole path.  Each GPU the library runs on holds its own copy at its
// own address until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address, so it is never handed to a kernel or a copy: the first call on a
// device looks the device address up once (hipGetSymbolAddress, with that
// device current) and every later use goes through that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dsa.h"
#include "kernels.hpp"

static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_WORKSPACE_BYTES];

namespace dsa {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t noalloc_workspace(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

}  // namespace dsa
