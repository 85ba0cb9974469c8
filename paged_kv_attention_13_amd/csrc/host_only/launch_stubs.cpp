// Kernel-launcher stand-ins for the host-only build of the library (g++, no HIP runtime):
// the argument checks, plans, metadata checkers, scheduler and block manager are the
// library's own sources, and every call that would reach a kernel launch returns the
// HIP "no device" error instead.  The sanitizer tests load that build.
#include "pa_internal.h"

namespace pa {
namespace {
constexpr int kNoDevice = 100;   // hipErrorNoDevice
}

int launch_decode_partials(const DecodeLaunch &, void *) { return kNoDevice; }
int launch_merge(const DecodeLaunch &, void *) { return kNoDevice; }
int launch_prefill(const PrefillLaunch &, void *) { return kNoDevice; }
int launch_prefill_merge(const PrefillLaunch &, void *) { return kNoDevice; }
int launch_append(const AppendLaunch &, void *) { return kNoDevice; }
int launch_verify_partials(const VerifyLaunch &, void *) { return kNoDevice; }
int launch_verify_merge(const VerifyLaunch &, void *) { return kNoDevice; }
int launch_cascade_merge(const CascadeMergeLaunch &, void *) { return kNoDevice; }
int launch_stream_read(const void *, size_t, uint32_t *, int, int, void *) { return kNoDevice; }
int launch_gather_read(const void *, const int64_t *, long long, int, uint32_t *, int, int, void *) { return kNoDevice; }
int fork_side_stream(void *, void **) { return kNoDevice; }
int static_scratch(void **) { return kNoDevice; }
int join_side_stream(void *) { return kNoDevice; }
unsigned int *device_check_flags() { return nullptr; }
int read_and_clear_check_flags(uint32_t *flags) {
  *flags = 0;
  return PA_DEVICE_CHECKS ? kNoDevice : 0;
}
const char *hip_error_name(int) { return "hipErrorNoDevice (host-only build)"; }

}  // namespace pa
