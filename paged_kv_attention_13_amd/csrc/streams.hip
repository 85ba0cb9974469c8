// One auxiliary stream per device, used to run a mixed batch's prefill-chunk
// rows (bound by the matrix cores) beside its decode rows (bound by HBM
// bandwidth): the two kernels use different units, so running them at the
// same time hides most of the shorter one.
//
// fork(main): an event recorded on `main` is waited for by the auxiliary
// stream, so work queued there next starts after everything already queued on
// `main`; join(main): `main` waits for an event recorded on the auxiliary
// stream, so work queued on `main` afterwards (and the caller) sees the
// auxiliary work complete.  Both are plain event record / wait operations, so
// a fork/join pair inside a stream capture joins the auxiliary stream to the
// capture.  The stream (default priority) and its two events are created on
// first use on each device and kept until the process ends.  Each record/wait
// pair runs under a per-device lock, so host threads sharing a device stay
// correctly ordered (their auxiliary work may then wait on each other).
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMaxDevices = 64;

struct SideStream {
  std::once_flag once;
  hipError_t status = hipSuccess;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  std::mutex lock;
};

SideStream g_side[kMaxDevices];

int side_for_current_device(SideStream **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  SideStream &s = g_side[dev];
  std::call_once(s.once, [&s]() {
    s.status = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking);
    if (s.status == hipSuccess) s.status = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming);
    if (s.status == hipSuccess) s.status = hipEventCreateWithFlags(&s.join, hipEventDisableTiming);
  });
  if (s.status != hipSuccess) return (int)s.status;
  *out = &s;
  return 0;
}

}  // namespace

int fork_side_stream(void *main_stream, void **side_stream) {
  SideStream *s = nullptr;
  int e = side_for_current_device(&s);
  if (e) return e;
  hipStream_t m = static_cast<hipStream_t>(main_stream);
  std::lock_guard<std::mutex> g(s->lock);
  hipError_t r = hipEventRecord(s->fork, m);
  if (r == hipSuccess) r = hipStreamWaitEvent(s->stream, s->fork, 0);
  if (r != hipSuccess) return (int)r;
  *side_stream = s->stream;
  return 0;
}

int join_side_stream(void *main_stream) {
  SideStream *s = nullptr;
  int e = side_for_current_device(&s);
  if (e) return e;
  hipStream_t m = static_cast<hipStream_t>(main_stream);
  std::lock_guard<std::mutex> g(s->lock);
  hipError_t r = hipEventRecord(s->join, s->stream);
  if (r == hipSuccess) r = hipStreamWaitEvent(m, s->join, 0);
  return (int)r;
}

}  // namespace pa
