// The library's one fixed device buffer: the workspace of orbq_linear_noalloc (token codes and
// norms, or the 6-bit path's bf16 centroids), for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; in host code its name is only a host-side stand-in,
// so the device address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to kernels.  Each GPU the library runs on holds
// its own copy of the array (ORBQ_NOALLOC_SCRATCH_BYTES) until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/orbq.h"
#include "internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[ORBQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace orbq {

// The device address of the current device's scratch array (looked up on the device's first
// call and kept).  Returns hipSuccess or the lookup's error.
int noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (!p) return static_cast<int>(hipErrorInvalidSymbol);
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return static_cast<int>(hipSuccess);
}

}  // namespace orbq
