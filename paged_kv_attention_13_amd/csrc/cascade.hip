// Final merge of a shared-prefix (cascade) decode call on gfx950.
//
// Rows that start with the same tokens point at the same cache blocks (prefix
// reuse: "How does TensorRT-LLM work", outcomeschool.com, section "The paged
// KV cache"; block reuse for a shared system prompt: "TensorRT-LLM, in depth",
// aicassindra.com, section "The paged KV cache and block reuse").  A group of
// consecutive decode rows sharing a prefix is attended over that prefix once,
// all its queries together (the prefix mode of the multi-query kernel), and
// each row over the rest of its own cache (the decode kernel with a per-row
// start).  Both leave log2-domain partials (m, l, acc) per piece; here the
// pieces of one (row, query head) are combined with the log-sum-exp identity
// -- the same merge that joins the pieces of a split context
// ("Introduction to TensorRT-LLM", dileepadev.github.io, section "Core
// Optimization Technologies", Flash-Decoding):
//     o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int D = kHeadDim;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One wave per (query head, row); each lane combines two of the 128 elements.
template <bool OUT_BF16>
__global__ __launch_bounds__(64) void cascade_merge_kernel(CascadeMergeLaunch p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int Hkv = p.num_kv_heads;
  const int G = p.num_q_heads / Hkv;
  const int g = h / G;
  const int hh = h % G;
  // the row's own part
  // piece records are clamped to the slots of the launches' workers, so a record that does
  // not come from this call's partials gives wrong numbers, never a read outside the workspace
  const int us = b * Hkv + g;
  const int fs = min(max(p.seg_first[us], 0), p.row_workers - 1);
  const int cs = min(max(p.seg_count[us], 0), p.row_workers - fs);
  // its group (last k with group_start[k] <= b) and its column in the group's prefix pieces
  int lo = 0, hi = p.num_groups;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.group_start[mid] <= b) lo = mid;
    else hi = mid;
  }
  const int up = lo * Hkv + g;
  const int col = min(max((b - p.group_start[lo]) * G + hh, 0), p.slot_cols - 1);
  const bool has_prefix = p.shared_len[b] > 0;
  const int fp = has_prefix ? min(max(p.pseg_first[up], 0), p.prefix_workers - 1) : 0;
  const int cp = has_prefix ? min(max(p.pseg_count[up], 0), p.prefix_workers - fp) : 0;

  // pieces 0 .. cs-1 are the row's own, cs .. cs+cp-1 the prefix's; lane i holds piece
  // i's (m, l) so that every piece's scalars load at once, then the 128-element
  // partials are combined piece by piece (all their addresses known up front)
  const int n = cs + cp;
  auto m_of = [&](int i) {
    return i < cs ? p.part_m[(size_t)(us + fs + i) * G + hh]
                  : p.ppart_m[(size_t)(up + fp + i - cs) * p.slot_cols + col];
  };
  auto l_of = [&](int i) {
    return i < cs ? p.part_l[(size_t)(us + fs + i) * G + hh]
                  : p.ppart_l[(size_t)(up + fp + i - cs) * p.slot_cols + col];
  };
  auto acc_of = [&](int i) {
    return i < cs ? p.part_acc + ((size_t)(us + fs + i) * G + hh) * D
                  : p.ppart_acc + ((size_t)(up + fp + i - cs) * p.slot_cols + col) * D;
  };
  float M = kNegBig;
  for (int base = 0; base < n; base += 64)
    if (base + lane < n) M = fmaxf(M, m_of(base + lane));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float den = 0.f, n0 = 0.f, n1 = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const float wt = i < n ? fast_exp2(m_of(i) - M) : 0.f;
    const float li = i < n ? l_of(i) : 0.f;
    const int cnt = min(64, n - base);
    // numerator and denominator accumulate in the same order (a constant V stays exact)
#pragma unroll 4
    for (int j = 0; j < cnt; ++j) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), j));
      const float lj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, li), j));
      const float2 a = *reinterpret_cast<const float2 *>(acc_of(base + j) + 2 * lane);
      den = __builtin_fmaf(w, lj, den);
      n0 = __builtin_fmaf(w, a.x, n0);
      n1 = __builtin_fmaf(w, a.y, n1);
    }
  }
  const size_t o = ((size_t)b * p.num_q_heads + h) * D + 2 * lane;
  if constexpr (OUT_BF16) {
    static_cast<__bf16 *>(p.out)[o] = (__bf16)(n0 / den);
    static_cast<__bf16 *>(p.out)[o + 1] = (__bf16)(n1 / den);
  } else {
    static_cast<float *>(p.out)[o] = n0 / den;
    static_cast<float *>(p.out)[o + 1] = n1 / den;
  }
}

}  // namespace

int launch_cascade_merge(const CascadeMergeLaunch &M, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  dim3 grid(M.num_q_heads, M.num_seqs);
  if (M.out_dtype == PA_BF16)
    hipLaunchKernelGGL(cascade_merge_kernel<true>, grid, dim3(64), 0, st, M);
  else
    hipLaunchKernelGGL(cascade_merge_kernel<false>, grid, dim3(64), 0, st, M);
  return (int)hipGetLastError();
}

}  // namespace pa
