// noalloc.hip -- the fixed device workspace of bsa_forward_noalloc, the entry
// point for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace is one file-scope device array.  Each device the library
// runs on holds its own copy for the life of the process.  In host code the
// array's name is only a host-side stand-in, so its device address is looked
// up once per device with hipGetSymbolAddress (with that device current, at
// handle creation) and only that address is ever passed to kernels.  Every
// call on a device shares the array: calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bsa_launch.hpp"

namespace bsa {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[device] = p;
  }
  *out = g_addr[device];
  return hipSuccess;
}

}  // namespace bsa
