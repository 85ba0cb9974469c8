// Device side of the debug builds' metadata checks (PA_DEVICE_CHECKS=1): each helper returns
// the value the kernel may use safely and, when the metadata broke its bound, ors a bit into
// the per-GPU flags word.  With the checks off the helpers return their argument unchanged.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

// One vector atomic, from the first active lane (a lane-divergent branch, so never a scalar
// memory operation).
__device__ __forceinline__ void report_check(unsigned int *flags, unsigned int bit) {
  const unsigned long long active = __builtin_amdgcn_ballot_w64(true);
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if (flags && lane == __builtin_ctzll(active))
    __hip_atomic_fetch_or(flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A block id read from the table: outside [0, num_blocks) -> block 0.
__device__ __forceinline__ int checked_block(int phys, int num_blocks, unsigned int *flags) {
#if PA_DEVICE_CHECKS
  if (phys < 0 || phys >= num_blocks) {
    report_check(flags, PA_CHECK_BLOCK_ID);
    return 0;
  }
#endif
  return phys;
}

// A row length: outside [1, max_len] -> clamped into it.
__device__ __forceinline__ int checked_len(int L, int max_len, unsigned int *flags) {
#if PA_DEVICE_CHECKS
  if (L < 1 || L > max_len) {
    report_check(flags, PA_CHECK_SEQ_LEN);
    return L < 1 ? 1 : max_len;
  }
#endif
  return L;
}

// A row's query count: outside [1, L] -> clamped into it.
__device__ __forceinline__ int checked_qlen(int n, int L, unsigned int *flags) {
#if PA_DEVICE_CHECKS
  if (n < 1 || n > L) {
    report_check(flags, PA_CHECK_Q_LEN);
    return n < 1 ? 1 : L;
  }
#endif
  return n;
}

// A row's queries [q_begin, q_begin + n) of the total_q rows of q: a range outside them ->
// the row's first query only (q_begin 0, n 1).
__device__ __forceinline__ void checked_qrange(int &q_begin, int &n, int L, int total_q, unsigned int *flags) {
#if PA_DEVICE_CHECKS
  n = checked_qlen(n, L, flags);
  if (q_begin < 0 || (long long)q_begin + n > total_q) {
    report_check(flags, PA_CHECK_Q_LEN);
    q_begin = 0;
    n = 1;
  }
#endif
}

// An append slot: at or past num_blocks * block_size -> -1 (the token is skipped).
__device__ __forceinline__ int checked_slot(int slot, int num_blocks, int block_size, unsigned int *flags) {
#if PA_DEVICE_CHECKS
  if (slot >= 0 && (long long)slot >= (long long)num_blocks * block_size) {
    report_check(flags, PA_CHECK_SLOT);
    return -1;
  }
#endif
  return slot;
}

}  // namespace pa
