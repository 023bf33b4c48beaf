// Library-owned device scratch for abatt_plan_noalloc: the plan workspace
// (key means, centroids, weights, scores, sampler scratch) for callers that
// cannot allocate device memory.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from the moment the code object is loaded on it
// until the process ends.  In host code `scratch` names a host-side shadow,
// not device memory: the device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is ever
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abatt.h"
#include "kernels.h"

namespace abatt {

static_assert(ABATT_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of 256 bytes");

static __device__ __align__(256) unsigned char scratch[ABATT_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace abatt
