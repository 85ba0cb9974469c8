// The flags word of debug builds (PA_DEVICE_CHECKS=1): the kernels or their metadata
// violations into it (a block id outside the pool, a row length outside [1, max_len], a
// query count outside [1, row length], an append slot outside the pool) and carry on with a
// safe value instead of reading or writing out of bounds; pa_device_check_flags reads and
// clears it.  One word per GPU (a file-scope __device__ variable), its device address looked
// up once per device with hipGetSymbolAddress, as for the static scratch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned int check_flags_word[64];

namespace {

constexpr int kMaxDevices = 64;

struct FlagsAddress {
  std::once_flag once;
  unsigned int *ptr = nullptr;
};

FlagsAddress g_flags[kMaxDevices];

unsigned int *flags_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  FlagsAddress &f = g_flags[dev];
  std::call_once(f.once, [&f]() {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_flags_word)) == hipSuccess) f.ptr = static_cast<unsigned int *>(p);
  });
  return f.ptr;
}

}  // namespace

unsigned int *device_check_flags() { return PA_DEVICE_CHECKS ? flags_address() : nullptr; }

int read_and_clear_check_flags(uint32_t *flags) {
  *flags = 0;
  if (!PA_DEVICE_CHECKS) return 0;
  unsigned int *p = flags_address();
  if (!p) return (int)hipErrorInvalidSymbol;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return (int)e;
  unsigned int v = 0;
  e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  e = hipMemset(p, 0, sizeof v);
  if (e != hipSuccess) return (int)e;
  e = hipDeviceSynchronize();
  *flags = v;
  return (int)e;
}

}  // namespace pa
