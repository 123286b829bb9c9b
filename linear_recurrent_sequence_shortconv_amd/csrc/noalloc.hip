// Fixed device array for the entry point that allocates nothing
// (prism_step_noalloc): callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid it) run the
// recurrent step with its refinement pairs in this array instead of a
// workspace of their own.
//
// The array is one file-scope __device__ variable: each GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol, so the device
// address is looked up once per device, with that device current, and kept;
// kernels and copies always receive that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "prism_internal.h"

namespace prism {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};
}  // namespace

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream); the lookup runs once per device, with
// that device made current for it.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace prism
