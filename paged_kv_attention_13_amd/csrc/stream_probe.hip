// Streaming-read probe: the achievable HBM read bandwidth with the decode kernels' load
// form (16-byte non-temporal loads, consecutive lanes on consecutive 16 bytes).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup w reads chunks w, w + grid, ... of kThreads * U consecutive 16-byte vectors,
// U loads in flight per lane (lane l takes vectors l, l + 256, ...: each load instruction
// covers 4 KB of consecutive bytes), then the vectors past the last whole chunk.
template <int U>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *src, size_t n, unsigned *out) {
  constexpr size_t kChunk = (size_t)kThreads * U;
  const size_t whole = n / kChunk * kChunk;
  unsigned acc = 0;
  for (size_t base = (size_t)blockIdx.x * kChunk; base < whole; base += (size_t)gridDim.x * kChunk) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(src + base + k * kThreads + threadIdx.x);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= fold(v[k]);
  }
  for (size_t i = whole + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
    acc ^= fold(__builtin_nontemporal_load(src + i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace
}  // namespace pa

namespace pa {

int launch_stream_read(const void *src, size_t bytes, uint32_t *out, int num_workgroups, int loads_in_flight,
                       void *stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4 *s = static_cast<const u32x4 *>(src);
  unsigned *o = reinterpret_cast<unsigned *>(out);
  const size_t n = bytes / 16;
  if (loads_in_flight == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(num_workgroups), dim3(kThreads), 0, st, s, n, o);
  else if (loads_in_flight == 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(num_workgroups), dim3(kThreads), 0, st, s, n, o);
  else
    hipLaunchKernelGGL(stream_read_kernel<16>, dim3(num_workgroups), dim3(kThreads), 0, st, s, n, o);
  return (int)hipGetLastError();
}

}  // namespace pa
