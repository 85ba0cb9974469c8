// Internal declarations shared by the host code (plain C++) and the HIP
// kernel files.  Nothing here is part of the public ABI (include/pa.h).
#ifndef PA_INTERNAL_H_
#define PA_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Shapes the kernels are compiled for.
constexpr int kHeadDim = 128;
constexpr int kWavesPerBlock = 4;        // decode kernel: 4 wave64 per workgroup
constexpr int kPartitionQuantum = 128;   // partition sizes are multiples of this
constexpr int kMaxPagesPerPartition = 64;  // one block-table entry per lane of a wave
constexpr int kTargetCUs = 256;          // MI355X compute units (grid planning only)

// Everything a decode launch needs, resolved on the host.
struct DecodeLaunch {
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const float *k_scale;
  const float *v_scale;
  const int32_t *block_table;
  const int32_t *seq_lens;
  void *out;
  float *part_m;      // [B][Hq][S]
  float *part_l;      // [B][Hq][S]
  float *part_acc;    // [B][Hq][S][D]
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  int partition_size;
  int num_partitions;
  int kv_dtype;
  int out_dtype;
  float scale;
};

struct PrefillLaunch {
  const void *q;                 // [total_q][Hq][D] bf16
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_table;
  const int32_t *seq_lens;
  const int32_t *q_start_loc;
  void *out;
  int first_row;                 // first prefill row
  int num_rows;                  // prefill rows
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  int max_q_len;
  int out_dtype;
  float scale;
};

// Host helpers (pa_host.cpp).
pa_status set_error(pa_status s, const char *fmt, ...);
pa_status validate_decode(const pa_decode_args *a, bool need_device_pointers);
pa_status plan_decode(const pa_decode_args *a, pa_plan *plan);
pa_status make_decode_launch(const pa_decode_args *a, const pa_plan &plan, DecodeLaunch *L);
size_t elem_bytes(int dtype);

// Kernel launchers (decode.hip, prefill.hip).  Return 0 on success, else the
// HIP error code of the failed launch.
int launch_decode_partials(const DecodeLaunch &L, void *stream);
int launch_merge(const DecodeLaunch &L, void *stream);
int launch_prefill(const PrefillLaunch &L, void *stream);
const char *hip_error_name(int code);

}  // namespace pa

#endif  // PA_INTERNAL_H_
