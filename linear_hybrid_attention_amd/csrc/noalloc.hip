// ttr_hybrid_forward_noalloc: the hybrid forward with its workspace in a
// fixed device array of this library instead of a caller's buffer, for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array (TTR_NOALLOC_SCRATCH_BYTES) is a file-scope __device__ object:
// every GPU the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the first call on a device, with that
// device current, asks HIP for the copy's device address once and keeps it
// per device; every launch takes that address. Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ttr.h"
#include "launch.hpp"

namespace {

__device__ __align__(256) unsigned char scratch[TTR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of this device's copy (NULL: not looked up yet)

// The current device's copy of the array, looked up on its first use.
ttr_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ttr::report_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return TTR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return ttr::report_hip(e);
    if (p == nullptr) return ttr::report_hip(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TTR_OK;
}

}  // namespace

extern "C" ttr_status ttr_hybrid_forward_noalloc(ttr_dims d, const void* Q, const void* K, const void* V,
                                                 const void* W, const float* b, const float* g, float eps,
                                                 int32_t L, int32_t causal, void* out, void* stream) {
  // the shape checks are ttr_hybrid_forward's; here only the size of the array
  if (ttr_workspace_bytes(d, L, causal, 0) > (size_t)TTR_NOALLOC_SCRATCH_BYTES) return TTR_ERR_WORKSPACE;
  void* ws = nullptr;
  const ttr_status st = scratch_of_current_device(&ws);
  if (st != TTR_OK) return st;
  return ttr_hybrid_forward(d, Q, K, V, W, b, g, eps, L, causal, out, ws, (size_t)TTR_NOALLOC_SCRATCH_BYTES, stream);
}
