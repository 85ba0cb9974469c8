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

// Paged gather: wave w reads pages [w * P / nw, (w + 1) * P / nw) of the list in order,
// each page `page_bytes` (a multiple of 1 KB) at base + offsets[i]: one 16-byte load per lane
// covers 1 KB of a page, with PF pages' kilobytes in flight.
template <int PF>
__global__ __launch_bounds__(kThreads) void gather_read_kernel(const char *base, const int64_t *offsets,
                                                               long long npages, int page_bytes, unsigned *out) {
  const int lane = threadIdx.x & 63;
  const long long nw = (long long)gridDim.x * (kThreads / 64);
  const long long w = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const long long p0 = w * npages / nw;
  const long long p1 = (w + 1) * npages / nw;
  const int kb = page_bytes >> 10;
  unsigned acc = 0;
  long long i = p0;
  for (; i + PF - 1 < p1; i += PF) {
    const char *pg[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) pg[k] = base + offsets[i + k] + 16 * lane;
    for (int c = 0; c < kb; ++c) {
      u32x4 v[PF];
#pragma unroll
      for (int k = 0; k < PF; ++k) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pg[k] + 1024 * c));
#pragma unroll
      for (int k = 0; k < PF; ++k) acc ^= fold(v[k]);
    }
  }
  for (; i < p1; ++i)
    for (int c = 0; c < kb; ++c)
      acc ^= fold(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + offsets[i] + 16 * lane + 1024 * c)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) out[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
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

int launch_gather_read(const void *base, const int64_t *offsets, long long npages, int page_bytes, uint32_t *out,
                       int num_workgroups, int pages_in_flight, void *stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char *b = static_cast<const char *>(base);
  unsigned *o = reinterpret_cast<unsigned *>(out);
  if (pages_in_flight == 2)
    hipLaunchKernelGGL(gather_read_kernel<2>, dim3(num_workgroups), dim3(kThreads), 0, st, b, offsets, npages, page_bytes, o);
  else if (pages_in_flight == 4)
    hipLaunchKernelGGL(gather_read_kernel<4>, dim3(num_workgroups), dim3(kThreads), 0, st, b, offsets, npages, page_bytes, o);
  else
    hipLaunchKernelGGL(gather_read_kernel<8>, dim3(num_workgroups), dim3(kThreads), 0, st, b, offsets, npages, page_bytes, o);
  return (int)hipGetLastError();
}

}  // namespace pa
