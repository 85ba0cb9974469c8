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
constexpr int kWavesPerBlock = 4;        // decode kernel: 4 independent wave64 workers per workgroup
constexpr int kDefaultCUs = 256;         // MI355X compute units: the plan's count where no
                                         // device can be asked (a host-only build)
// Compute units of the current device, read once per device (device_info.hip).
int device_cus();
// decode kernel: one wave per SIMD (4 per CU) ...
inline int decode_max_workers(int cus) { return cus * 4; }
constexpr int kShortUnitTiles = 32;      // ... or two when no unit (row, kv head) exceeds this
                                         // many tiles: short units are bound by their start-up
                                         // latency, which more resident waves overlap
constexpr int kMinTilesPerWorker = 4;    // below this, fewer workers are launched
constexpr int kCascadeRowMinTiles = 12;  // shared-prefix calls, row parts: every piece is a
                                         // partial, so pieces are kept longer
constexpr int kCascadePrefixMinTiles = 2;   // shared-prefix calls, prefix part: few, long units;
                                            // more workers hide their start-up latency
constexpr int kVerifyTile = 32;          // verify kernel: tokens per tile
constexpr int kVerifyMaxCols = 32;       // verify kernel: query columns (q_len x group) per kv head
inline int verify_max_workers(int cus) { return cus * 4; }   // one verify wave per SIMD
constexpr int kMqUnitCost = 2;           // multi-query kernel: start-up cost of a unit, in tiles
                                         // (FP8 rows of 128-8,192 tokens: 2 measured best of 0-4)
constexpr int kDecodeUnitCost = 4;       // decode kernel: start-up cost of a unit, in 16-token
                                         // tiles (measured: each unit a wave starts delays its
                                         // end by ~4.5 us, the time of ~3.6 tiles)
constexpr int kUnitMaxTokens = 1024;     // decode: rows bounded by this many tokens (and 64
                                         // pages) run one workgroup per (row, kv head) unit
// ... when there are at most two units per CU (512 on 256 CUs); beyond it the balanced
// split measured 16-29 % faster
inline int unit_max_units(int cus) { return cus * 2; }
// waves of that workgroup: 8, or 4 where the per-wave state is large (fp32 pools,
// or 8 query heads per kv head), which then fits one wave per SIMD without spills
constexpr int unit_waves(int kv_dtype, int group) { return (kv_dtype == PA_F32 || group >= 8) ? 4 : 8; }
// Prefill workgroup shapes: 4 waves staging 64-token kv tiles, two workgroups per CU; or 8
// waves staging 128-token tiles, one workgroup per CU (each staged tile and barrier serve twice
// the queries).  Both compute 64-token sub-tiles.
inline int prefill_tile(int waves) { return 16 * waves; }                       // kv tokens per staged tile
inline int prefill_slots(int cus, int waves) { return waves == 4 ? cus * 2 : cus; }  // resident workgroups
constexpr int kPrefillMaxSplits = 8;     // prefill: at most this many kv pieces per unit
constexpr int kPrefillMinChunkTiles = 4; // prefill: a piece covers at least this many tiles

// Prefill geometry for group size G: query heads per workgroup (HB) and query
// positions per workgroup (QB); a unit is (row, kv head, head block, query tile).
inline int prefill_heads_per_block(int G) { return G == 1 ? 1 : (G == 2 ? 2 : 4); }
inline int prefill_queries_per_block(int G, int waves) { return 32 * (waves / prefill_heads_per_block(G)); }

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
  int32_t *seg_first;  // [B*Hkv] first worker covering each (row, kv head) unit
  int32_t *seg_count;  // [B*Hkv] number of workers covering it
  float *part_m;       // [(B*Hkv + workers) * G]   partial slot (unit + worker), head in group
  float *part_l;       // same
  float *part_acc;     // [(B*Hkv + workers) * G][D]
  const int32_t *kv_start;   // [B] first token each row covers (multiple of bs), or null for 0;
                             // when set, every piece (whole units too) is left as a partial
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  // debug builds (PA_DEVICE_CHECKS=1): the metadata bounds the kernels check at each use,
  // and the device word their violations are or-ed into (null in other builds)
  int num_blocks;
  int max_len;                   // min(max_seq_len, max_blocks_per_seq * block_size)
  int total_q;                   // rows of q and out
  unsigned int *check_flags;
  int num_workers;
  int workers_auto;    // 1 when the library chose num_workers (the kernel may use fewer)
  int min_tiles;       // with workers_auto: at least this many tiles per worker (the plan
                       // only knows an upper bound of the row lengths)
  int unit_cost;       // virtual tiles charged per unit in the work split
  int kv_dtype;
  int out_dtype;
  float scale;
  int unit_mode;       // 1: one workgroup per (row, kv head) unit, merged in LDS
  int unit_pieces;     // unit mode: workgroups per unit; 1 = no workspace, no merge, else each
                       // writes the partial of its share of the unit's tiles to slot
                       // unit * unit_pieces + piece and the merge kernel combines them
  // fused append (unit mode only): row b's new token k_new/v_new[b] ([B][Hkv][D], the pool
  // dtype) is written to slot new_slots[b] (-1: none) of the pools, and used for position
  // seq_len - 1 instead of reading that slot
  const void *k_new;
  const void *v_new;
  const int32_t *new_slots;
  void *k_pool_w;
  void *v_pool_w;
};

struct PrefillLaunch {
  const void *q;                 // [total_q][Hq][D] bf16
  const void *k_pool;            // bf16 or FP8-E4M3 pools
  const void *v_pool;
  const float *k_scale;          // [Hkv] FP8 pools: dequantisation scales (else unused)
  const float *v_scale;
  int kv_dtype;                  // PA_BF16 or PA_FP8_E4M3
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
  // debug builds (PA_DEVICE_CHECKS=1): the metadata bounds the kernels check at each use,
  // and the device word their violations are or-ed into (null in other builds)
  int num_blocks;
  int max_len;                   // min(max_seq_len, max_blocks_per_seq * block_size)
  int total_q;                   // rows of q and out
  unsigned int *check_flags;
  int max_q_len;
  int out_dtype;
  float scale;
  // kv split of long units: every unit's tiles are cut into pieces of C tiles
  // (C computed in the kernel from the rows' lengths, at least ceil(tiles / splits));
  // pieces of a cut unit go to per-(unit, piece) slots and a merge kernel combines them
  int splits;                    // 1 = no split
  int max_qtiles;                // ceil(max_q_len / QB)
  int resident_slots;            // prefill workgroups resident at once on the device
  int waves;                     // workgroup shape: 4 or 8 waves (32 query positions each)
  float *part_o;                 // [slot][waves][32 q][128] fp32, unnormalised
  float *part_ml;                // [slot][waves][32 q][2] fp32: running max (log2 domain), sum
};

struct VerifyLaunch {
  const void *q;                 // [total_q][Hq][D] bf16
  const void *k_pool;            // bf16 or FP8 pools
  const void *v_pool;
  const int32_t *block_table;
  const int32_t *seq_lens;
  const int32_t *q_start_loc;
  void *out;
  int32_t *seg_first;            // [rows*Hkv] first worker covering each (row, kv head) unit
  int32_t *seg_count;            // [rows*Hkv] number of workers covering it
  float *part_m;                 // [(rows*Hkv + workers) * slot_cols] partial slot (unit + worker), column
  float *part_l;
  float *part_acc;               // [... * slot_cols][D]
  const int32_t *group_start;    // prefix mode: [num_rows + 1] rows of each group
  const int32_t *shared_len;     // prefix mode: [B] shared prefix tokens of each row
  const float *k_scale;          // [Hkv] (FP8 pools only)
  const float *v_scale;
  int item_kind;                 // 0: items are verify rows (causal, own cache);
                                 // 1: items are groups of decode rows over their shared prefix
                                 //    (no mask inside the prefix; every piece left as a partial);
                                 // 2: items are decode rows (one query each, at the row index)
  int kv_dtype;                  // PA_BF16 or PA_FP8_E4M3
  int first_row;                 // first verify row (verify mode)
  int num_rows;                  // items: verify rows, or groups
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  // debug builds (PA_DEVICE_CHECKS=1): the metadata bounds the kernels check at each use,
  // and the device word their violations are or-ed into (null in other builds)
  int num_blocks;
  int max_len;                   // min(max_seq_len, max_blocks_per_seq * block_size)
  int total_q;                   // rows of q and out
  unsigned int *check_flags;
  int num_workers;
  int workers_auto;              // 1 when the library chose num_workers (the kernel may use fewer)
  int min_tiles;                 // with workers_auto: at least this many tiles per worker
  int slot_cols;                 // max_verify_q_len * G (<= kVerifyMaxCols)
  int unit_cost;                 // virtual tiles charged per unit in the work split
  int out_dtype;
  float scale;
};

// Final merge of a shared-prefix decode call: for every (row, query head), the
// pieces of the row's own part (decode-kernel partials, slot (unit + worker) * G + head)
// and of its group's shared prefix (prefix-kernel partials, slot (unit + worker) *
// slot_cols + column).
struct CascadeMergeLaunch {
  const int32_t *group_start;
  const int32_t *shared_len;
  const int32_t *seg_first;      // row parts: [B*Hkv]
  const int32_t *seg_count;
  const float *part_m;
  const float *part_l;
  const float *part_acc;
  const int32_t *pseg_first;     // prefixes: [groups*Hkv]
  const int32_t *pseg_count;
  const float *ppart_m;
  const float *ppart_l;
  const float *ppart_acc;
  void *out;
  int num_seqs;
  int num_groups;
  int num_q_heads;
  int num_kv_heads;
  int slot_cols;
  int out_dtype;
  int row_workers;               // workers of the row-part launch (its slots: units + workers)
  int prefix_workers;            // workers of the prefix launch
};

struct AppendLaunch {
  const void *k;                 // [T][Hkv][D] src_dtype
  const void *v;
  const int32_t *slot_mapping;   // [T]
  void *k_pool;                  // [num_blocks][Hkv][bs][D] kv_dtype
  void *v_pool;
  const float *k_scale;          // [Hkv] (FP8 only)
  const float *v_scale;
  int num_tokens;
  int num_kv_heads;
  int block_size;
  int src_dtype;
  int kv_dtype;
  int num_blocks;                // debug builds: slots must lie below num_blocks * block_size
  unsigned int *check_flags;     // debug builds: violations or-ed here (else null)
};

// Debug builds compiled with PA_DEVICE_CHECKS=1 check the device-resident metadata at each
// use (block ids, row lengths, query counts, append slots) and record violations in a per-device
// flags word instead of reading or writing out of bounds; other builds compile the checks out.
#ifndef PA_DEVICE_CHECKS
#define PA_DEVICE_CHECKS 0
#endif
// The flags word of the current device (device address), or null when the checks are off or
// the address cannot be obtained (device_checks.hip).
unsigned int *device_check_flags();
// Synchronises the current device, returns its flags word and clears it (0 when the checks
// are off); a HIP error code or 0.
int read_and_clear_check_flags(uint32_t *flags);

// Host helpers (pa_host.cpp).
pa_status set_error(pa_status s, const char *fmt, ...);
int max_len_of(const pa_decode_args *a);
pa_status validate_decode(const pa_decode_args *a, bool need_device_pointers);
pa_status plan_decode(const pa_decode_args *a, pa_plan *plan);
pa_status make_decode_launch(const pa_decode_args *a, const pa_plan &plan, DecodeLaunch *L);
pa_status validate_append(const pa_append_args *a, bool need_device_pointers);
// pa_append_decode: both argument sets valid, one new token per decode row, same pools.
pa_status check_append_decode_pair(const pa_append_args *app, const pa_decode_args *dec,
                                   bool need_device_pointers);
size_t elem_bytes(int dtype);
// Sub-plans of a pa_mixed call: decode rows, verify rows, prefill rows.  Workspace:
// decode part first, then the verify part at verify_offset, then the prefill
// pieces at prefill_offset (only when prefill_splits > 1).
struct MixedPlan {
  pa_decode_args dec;
  pa_plan dec_plan;
  int verify_workers = 0;
  size_t verify_offset = 0;
  int prefill_splits = 1;
  int prefill_waves = 4;          // prefill workgroup shape (prefill_tile, prefill_slots)
  int prefill_qtiles = 0;
  size_t prefill_offset = 0;      // piece outputs
  size_t prefill_ml_offset = 0;   // piece (max, sum) pairs
  size_t prefill_slots = 0;
  size_t total_bytes = 0;
  int cus = kDefaultCUs;          // compute units the plan was made for
};
// Checks the pa_mixed row classes and fills the plan.
pa_status plan_mixed(const pa_mixed_args *a, bool need_device_pointers, MixedPlan *mp);
pa_status make_verify_launch(const pa_mixed_args *a, int workers, size_t verify_offset,
                             VerifyLaunch *V);
// Decode rows whose pools are FP8 run on the multi-query kernel (one query column per
// head); this builds that launch over the decode workspace layout.
pa_status make_decode_mq_launch(const pa_decode_args *a, const pa_plan &plan, VerifyLaunch *V);
inline bool decode_on_mq(const pa_decode_args *a) { return a->kv_dtype == PA_FP8_E4M3; }
// Short rows with the worker count left to the library: one workgroup per unit
// (every row within the first 64 block-table entries and kUnitMaxTokens tokens, at most
// two units per CU).
inline bool decode_unit_mode(const pa_decode_args *a, int cus) {
  return a->num_workers == 0 && a->num_seqs > 0 && a->kv_dtype != PA_FP8_E4M3 &&
         a->max_seq_len <= kUnitMaxTokens && a->max_seq_len <= 64 * a->block_size &&
         (int64_t)a->num_seqs * a->num_kv_heads <= unit_max_units(cus);
}
// Unit mode with few units: each unit's tiles are cut over this many workgroups, so that
// more CUs than units stream the cache (a unit's workgroup alone is bound by what one CU
// keeps in flight); at most one per CU in all, at least kUnitPieceTiles tiles each, and at
// most 8, which the merge reads in one round trip (a 546-token row: 9 pieces 14.0 us per call,
// 8 pieces 13.7 us; the 32-layer decode loop 0.383 -> 0.375 ms).
constexpr int kUnitPieceTiles = 4;
constexpr int kUnitMaxPieces = 8;
inline int decode_unit_pieces(const pa_decode_args *a, int cus) {
  const int64_t units = (int64_t)a->num_seqs * a->num_kv_heads;
  const int64_t tiles = (a->max_seq_len + 15) / 16;        // decode tiles (fp32 and bf16 pools)
  int64_t s = units > 0 ? cus / units : 1;
  if (s > (tiles + kUnitPieceTiles - 1) / kUnitPieceTiles) s = (tiles + kUnitPieceTiles - 1) / kUnitPieceTiles;
  if (s > kUnitMaxPieces) s = kUnitMaxPieces;
  return s >= 2 ? (int)s : 1;
}
// Resident multi-query waves: one per SIMD, two for FP8 pools with <= 16 columns.
inline int mq_max_workers(int kv_dtype, int slot_cols, int cus) {
  return (kv_dtype == PA_FP8_E4M3 && slot_cols <= 16) ? 2 * verify_max_workers(cus) : verify_max_workers(cus);
}
// Checks a shared-prefix decode call and resolves its three launches (prefix kernel,
// row-part decode kernel, final merge) over the caller's workspace; with
// need_device_pointers false only the sizes are computed.
pa_status plan_cascade(const pa_cascade_args *a, bool need_device_pointers, DecodeLaunch *dec,
                       VerifyLaunch *pre, CascadeMergeLaunch *mrg, size_t *total_bytes);
int tile_tokens(int kv_dtype);

// Kernel launchers (decode.hip, prefill.hip, verify.hip, append.hip).  Return 0 on success, else the
// HIP error code of the failed launch.
int launch_decode_partials(const DecodeLaunch &L, void *stream);
int launch_merge(const DecodeLaunch &L, void *stream);
int launch_prefill(const PrefillLaunch &L, void *stream);
int launch_prefill_merge(const PrefillLaunch &L, void *stream);
int launch_append(const AppendLaunch &L, void *stream);
int launch_verify_partials(const VerifyLaunch &V, void *stream);
int launch_verify_merge(const VerifyLaunch &V, void *stream);
int launch_cascade_merge(const CascadeMergeLaunch &M, void *stream);
int launch_stream_read(const void *src, size_t bytes, uint32_t *out, int num_workgroups, int loads_in_flight,
                       void *stream);
int launch_gather_read(const void *base, const int64_t *offsets, long long npages, int page_bytes, uint32_t *out,
                       int num_workgroups, int pages_in_flight, void *stream);
// The library's static scratch (static_scratch.hip): 16 MiB per device, used by
// pa_decode_noalloc in place of a caller workspace.  static_scratch() gives the current
// device's copy's device address (looked up once per device); returns 0 or a HIP error.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
int static_scratch(void **ptr);
// Auxiliary stream of the current device (streams.hip): fork makes it wait for the work
// queued so far on main_stream; join makes main_stream wait for the work queued on it.
int fork_side_stream(void *main_stream, void **side_stream);
int join_side_stream(void *main_stream);
const char *hip_error_name(int code);

}  // namespace pa

#endif  // PA_INTERNAL_H_
