// tern_noalloc.hip -- the static device scratch of tern_linear_noalloc, the
// variant of tern_linear for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the array's name stands for a host-side shadow, not a device address,
// so the host never passes it to a kernel: the first call on each device
// resolves the device address with hipGetSymbolAddress (that device
// current) and keeps it per device; every later use (the kernels' workspace
// argument) takes that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tern_internal.h"

namespace tern {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device ordinal

}  // namespace

int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

}  // namespace tern
