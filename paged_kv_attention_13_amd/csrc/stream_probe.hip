// Streaming-read probe: the achievable HBM read bandwidth with the decode kernels' load
// form (16-byte non-temporal loads, consecutive lanes on consecutive 16 bytes).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *src, size_t n, unsigned *out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  unsigned acc = 0;
  // four independent loads in flight per lane
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n; i += stride) acc ^= fold(__builtin_nontemporal_load(src + i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace
}  // namespace pa

namespace pa {

int launch_stream_read(const void *src, size_t bytes, uint32_t *out, int num_workgroups, void *stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4 *>(src), bytes / 16, reinterpret_cast<unsigned *>(out));
  return (int)hipGetLastError();
}

}  // namespace pa
