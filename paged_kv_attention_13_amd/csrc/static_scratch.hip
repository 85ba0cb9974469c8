// The library's static scratch: a fixed device array that pa_decode_noalloc uses for
// the split partials instead of a caller workspace, for callers that cannot allocate.
//
// The array is a file-scope __device__ variable: each GPU the library runs on holds its
// own copy, at its own address, until the process ends.  Host code never uses the
// variable's name as an address (on the host it is only a stand-in); the device address
// is looked up here once per device with hipGetSymbolAddress, with that device current,
// and kept.  Every call on one GPU shares that GPU's array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchAddress {
  std::once_flag once;
  hipError_t status = hipSuccess;
  void *ptr = nullptr;
};

ScratchAddress g_scratch[kMaxDevices];

}  // namespace

int static_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  ScratchAddress &s = g_scratch[dev];
  std::call_once(s.once, [&s]() {
    void *p = nullptr;
    s.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.status == hipSuccess && p == nullptr) s.status = hipErrorInvalidSymbol;
    s.ptr = p;
  });
  if (s.status != hipSuccess) return (int)s.status;
  *ptr = s.ptr;
  return 0;
}

}  // namespace pa
