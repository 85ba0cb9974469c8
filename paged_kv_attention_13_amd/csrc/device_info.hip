// Device properties the host plan uses, read once per device with that device
// current and kept until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  std::once_flag once;
  int cus = kDefaultCUs;
};

DeviceInfo g_info[kMaxDevices];

}  // namespace

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount).  The
// worker counts of the split (one or two waves per SIMD), the one-workgroup-per-unit
// limit and the prefill piece sizes scale with it.  Where the device cannot be asked,
// the MI355X count.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
  DeviceInfo &d = g_info[dev];
  std::call_once(d.once, [&d, dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) d.cus = n;
  });
  return d.cus;
}

}  // namespace pa
