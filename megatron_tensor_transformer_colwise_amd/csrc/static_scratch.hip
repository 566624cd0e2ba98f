// A fixed device array that serves as the attention sublayer's workspace for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// Each device the library runs on holds its own copy of the array from the
// first call on that device until the process ends.  Its device address is
// looked up once per device, with that device current, and cached; kernels
// only ever receive that address (the array's name in host code is a
// host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

static __device__ __align__(256) char scratch[tpk::kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of scratch on each device, once looked up
unsigned g_epoch[kMaxDevices];  // last epoch handed out for the flags at the start of scratch

}  // namespace

namespace tpk {

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
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

hipError_t static_scratch_epoch(unsigned* epoch) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  *epoch = ++g_epoch[dev];
  if (*epoch == 0) *epoch = ++g_epoch[dev];  // 0 is the flags' initial value (the array starts zeroed)
  return hipSuccess;
}

}  // namespace tpk
