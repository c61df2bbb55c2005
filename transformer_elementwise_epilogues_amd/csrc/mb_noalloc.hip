// mb_noalloc.hip -- the static device scratch behind the entry point that
// allocates nothing (mb_bias_gelu_bwd_noalloc).
//
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation) get the bias
// gradient's partial rows from a fixed array in the library's own device
// memory instead of a caller-provided workspace. Every GPU the library runs
// on holds its own copy of the array, at its own address, until the process
// ends. In host code the array's name is only a host-side stand-in, so the
// device address of each GPU's copy is looked up once (hipGetSymbolAddress,
// with that device current) and only that address is ever handed to kernels.
#include <mutex>

#include "mb_launch.hpp"

static __device__ __align__(256) unsigned char scratch[MB_NOALLOC_SCRATCH_BYTES];

namespace mb {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  // the device the work is enqueued on (the current device for the null stream)
  if (hipError_t e = hipStreamGetDevice(s, &dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipError_t e = hipGetDevice(&cur)) return e;
    if (cur != dev)
      if (hipError_t e = hipSetDevice(dev)) return e;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess && r != hipSuccess) return r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mb
