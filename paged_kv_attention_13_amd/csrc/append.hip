// Paged KV append on gfx950: write a step's new K/V tokens into their cache slots.
//
// Each step adds one key and one value vector per new token to its request's
// cache, in the request's current block or in a freshly handed-out one ("How
// does TensorRT-LLM work", outcomeschool.com, section "The paged KV cache";
// the scheduler of "TensorRT-LLM, in depth", aicassindra.com, section
// "In-flight batching and the scheduler", secures the room before the pass).
// The host's allocator decides where each token goes; the kernel receives one
// slot number per token, slot = block * block_size + offset, and -1 for a
// token to skip.  For an FP8 cache the code stored is E4M3(x / scale[g]): the
// quotient is an fp32 division, saturated to +-448 before the hardware's
// round-to-nearest-even conversion ("TensorRT-LLM, in depth", section
// "Quantization: fewer bytes per weight and per cached token", only says the
// cache may be FP8; saturation and rounding are this library's reading).
//
// One thread moves 8 consecutive elements of one (token, kv head) row:
// 16 threads cover a 128-element row, so loads and stores of a wave are
// contiguous 256-byte (bf16) rows; a bandwidth-bound scatter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "checks.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

constexpr int D = kHeadDim;
constexpr int kThreads = 256;
constexpr float kFp8Max = 448.0f;

template <int SRC>
__device__ __forceinline__ void load8(const void *base, size_t idx, float (&x)[8]) {
  if constexpr (SRC == PA_F32) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + idx);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + idx + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ai = a[i], bi = b[i];
      x[i] = __builtin_bit_cast(float, ai);
      x[4 + i] = __builtin_bit_cast(float, bi);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = a[i];
      x[2 * i] = __builtin_bit_cast(float, w << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
    }
  }
}

// two values -> two E4M3 codes packed into 16 bits
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  const i16x2 old = {0, 0};
  const i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

template <int SRC, int DST>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendLaunch p) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)p.num_tokens * p.num_kv_heads * (D / 8);
  if (i >= total) return;
  const int chunk = (int)(i & 15);
  const size_t th = i >> 4;
  const int g = (int)(th % p.num_kv_heads);
  const int t = (int)(th / p.num_kv_heads);
  const int slot = checked_slot(p.slot_mapping[t], p.num_blocks, p.block_size, p.check_flags);
  if (slot < 0) return;
  const int log2bs = __builtin_ctz(p.block_size);
  const int blk = slot >> log2bs;
  const int off = slot & (p.block_size - 1);
  const size_t src = ((size_t)t * p.num_kv_heads + g) * D + chunk * 8;
  const size_t dst = (((size_t)blk * p.num_kv_heads + g) * p.block_size + off) * D + chunk * 8;

  if constexpr (DST == SRC) {
    constexpr int EB = SRC == PA_F32 ? 4 : 2;
    const char *ks = static_cast<const char *>(p.k) + src * EB;
    const char *vs = static_cast<const char *>(p.v) + src * EB;
    char *kd = static_cast<char *>(p.k_pool) + dst * EB;
    char *vd = static_cast<char *>(p.v_pool) + dst * EB;
#pragma unroll
    for (int j = 0; j < EB / 2; ++j) {
      *reinterpret_cast<u32x4 *>(kd + 16 * j) = *reinterpret_cast<const u32x4 *>(ks + 16 * j);
      *reinterpret_cast<u32x4 *>(vd + 16 * j) = *reinterpret_cast<const u32x4 *>(vs + 16 * j);
    }
  } else {
    static_assert(DST == PA_FP8_E4M3, "conversions: same dtype, or to FP8");
    const float ksc = p.k_scale[g];
    const float vsc = p.v_scale[g];
    float x[8], y[8];
    load8<SRC>(p.k, src, x);
    load8<SRC>(p.v, src, y);
    uint32_t kw[2], vw[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float a[4], b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = fminf(fmaxf(x[4 * w + e] / ksc, -kFp8Max), kFp8Max);
        b[e] = fminf(fmaxf(y[4 * w + e] / vsc, -kFp8Max), kFp8Max);
      }
      kw[w] = enc2(a[0], a[1]) | (enc2(a[2], a[3]) << 16);
      vw[w] = enc2(b[0], b[1]) | (enc2(b[2], b[3]) << 16);
    }
    *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(p.k_pool) + dst) = u32x2{kw[0], kw[1]};
    *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(p.v_pool) + dst) = u32x2{vw[0], vw[1]};
  }
}

}  // namespace

int launch_append(const AppendLaunch &L, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t total = (size_t)L.num_tokens * L.num_kv_heads * (D / 8);
  if (total == 0) return 0;
  dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  if (L.kv_dtype == PA_FP8_E4M3) {
    if (L.src_dtype == PA_BF16)
      hipLaunchKernelGGL((append_kernel<PA_BF16, PA_FP8_E4M3>), grid, dim3(kThreads), 0, st, L);
    else
      hipLaunchKernelGGL((append_kernel<PA_F32, PA_FP8_E4M3>), grid, dim3(kThreads), 0, st, L);
  } else if (L.kv_dtype == PA_BF16) {
    hipLaunchKernelGGL((append_kernel<PA_BF16, PA_BF16>), grid, dim3(kThreads), 0, st, L);
  } else {
    hipLaunchKernelGGL((append_kernel<PA_F32, PA_F32>), grid, dim3(kThreads), 0, st, L);
  }
  return (int)hipGetLastError();
}

}  // namespace pa
