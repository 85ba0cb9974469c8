// Host side of the C ABI: argument validation, split-K planning, metadata
// checks and error reporting.  Plain C++ (no HIP calls) so that it can be
// built and tested on a machine without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2_block(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

// the longest row a call's metadata allows (the checked builds' bound on seq_lens)
int max_len_of(const pa_decode_args *a) {
  return (int)std::min<int64_t>(a->max_seq_len, (int64_t)a->max_blocks_per_seq * a->block_size);
}

pa_status set_error(pa_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(pa_status_string(s)) + ": " + buf;
  return s;
}

size_t elem_bytes(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

pa_status validate_decode(const pa_decode_args *a, bool need_device_pointers) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  if (a->num_seqs < 0) return set_error(PA_ERR_BAD_SHAPE, "num_seqs = %d < 0", a->num_seqs);
  if (a->num_kv_heads < 1 || a->num_q_heads < 1)
    return set_error(PA_ERR_BAD_SHAPE, "head counts must be >= 1 (Hq=%d, Hkv=%d)",
                     a->num_q_heads, a->num_kv_heads);
  if (a->num_q_heads % a->num_kv_heads != 0)
    return set_error(PA_ERR_BAD_SHAPE, "Hq=%d is not a multiple of Hkv=%d", a->num_q_heads,
                     a->num_kv_heads);
  const int group = a->num_q_heads / a->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return set_error(PA_ERR_UNSUPPORTED, "group size Hq/Hkv=%d (supported: 1, 2, 4, 8)", group);
  if (a->head_dim != kHeadDim)
    return set_error(PA_ERR_UNSUPPORTED, "head_dim=%d (supported: %d)", a->head_dim, kHeadDim);
  if (!is_pow2_block(a->block_size))
    return set_error(PA_ERR_UNSUPPORTED, "block_size=%d (supported: 16, 32, 64, 128)",
                     a->block_size);
  if (a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return set_error(PA_ERR_BAD_SHAPE, "num_blocks=%d, max_blocks_per_seq=%d must be >= 1",
                     a->num_blocks, a->max_blocks_per_seq);
  if (a->num_seqs > 0 && a->max_seq_len < 1)
    return set_error(PA_ERR_BAD_SHAPE, "max_seq_len=%d must be >= 1", a->max_seq_len);
  if ((int64_t)a->max_seq_len > (int64_t)a->max_blocks_per_seq * a->block_size)
    return set_error(PA_ERR_BAD_SHAPE, "max_seq_len=%d exceeds max_blocks_per_seq*block_size=%lld",
                     a->max_seq_len, (long long)a->max_blocks_per_seq * a->block_size);
  // dtype combinations
  const bool ok_out = a->out_dtype == PA_F32 || a->out_dtype == PA_BF16;
  bool ok = ok_out && ((a->q_dtype == PA_F32 && a->kv_dtype == PA_F32) ||
                       (a->q_dtype == PA_BF16 && a->kv_dtype == PA_BF16) ||
                       (a->q_dtype == PA_BF16 && a->kv_dtype == PA_FP8_E4M3));
  if (!ok)
    return set_error(PA_ERR_BAD_DTYPE,
                     "unsupported (q, kv, out) dtypes (%d, %d, %d); supported: (f32, f32, f32|bf16), "
                     "(bf16, bf16, bf16|f32), (bf16, fp8_e4m3, bf16|f32)",
                     a->q_dtype, a->kv_dtype, a->out_dtype);
  const bool fp8 = a->kv_dtype == PA_FP8_E4M3;
  if (!fp8 && (a->k_scale || a->v_scale))
    return set_error(PA_ERR_BAD_DTYPE, "k_scale/v_scale are only used with an FP8 KV cache");
  if (a->num_workers < 0 || a->num_workers > 65536)
    return set_error(PA_ERR_UNSUPPORTED, "num_workers=%d outside [0, 65536]", a->num_workers);
  if (need_device_pointers && a->num_seqs > 0) {
    if (!a->q || !a->k_pool || !a->v_pool || !a->block_table || !a->seq_lens || !a->out)
      return set_error(PA_ERR_NULL_POINTER, "q, k_pool, v_pool, block_table, seq_lens and out are required");
    if (fp8 && (!a->k_scale || !a->v_scale))
      return set_error(PA_ERR_NULL_POINTER, "an FP8 KV cache needs k_scale and v_scale");
    if (!aligned16(a->q) || !aligned16(a->k_pool) || !aligned16(a->v_pool) || !aligned16(a->out))
      return set_error(PA_ERR_MISALIGNED, "q, k_pool, v_pool and out must be 16-byte aligned");
    if (a->workspace && !aligned16(a->workspace))
      return set_error(PA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    // the kernels take the running maximum over unscaled scores (prefill) or fold the
    // scale into exp2 arguments: both need a positive, finite scale
    if (!(a->scale > 0.0f) || !std::isfinite(a->scale))
      return set_error(PA_ERR_UNSUPPORTED, "scale=%g must be finite and > 0", (double)a->scale);
  }
  return PA_OK;
}

int tile_tokens(int kv_dtype) { return kv_dtype == PA_FP8_E4M3 ? 32 : 16; }

// Weak default for builds without the HIP runtime (the host-only test build); the
// library's device_info.hip provides the real query.
__attribute__((weak)) int device_cus() { return kDefaultCUs; }

pa_status plan_decode(const pa_decode_args *a, pa_plan *plan) {
  const int tile = tile_tokens(a->kv_dtype);
  const int cus = device_cus();
  const int max_workers = decode_max_workers(cus);
  int nw = a->num_workers;
  if (nw == 0) {
    // One wave per SIMD (whole workgroups, one per CU) when units can be long: measured equal
    // to or 2-26 % faster than two waves per SIMD from units of 64 to 2,048 tiles (a single
    // 32,768-token row: 40.5 vs 55 us).  Two waves per SIMD when every unit is short (at most
    // 32 tiles): 3-9 % faster (2,048 rows of 128 tokens: 233 vs 251 us), the start-ups of more
    // units overlapping.  At least a few tiles per worker.  FP8 pools run on the multi-query
    // kernel (one column per query head), with its own resident-wave count.
    const int64_t units = (int64_t)a->num_seqs * a->num_kv_heads;
    const int64_t unit_tiles = (a->max_seq_len + tile - 1) / tile;
    const bool fp8 = a->kv_dtype == PA_FP8_E4M3;
    // the decode kernel's split also counts each unit's virtual start-up tiles
    const int64_t tiles_upper = units * (unit_tiles + (fp8 ? 0 : kDecodeUnitCost));
    const bool short_units = !fp8 && unit_tiles <= kShortUnitTiles;
    const int cap = fp8 ? mq_max_workers(a->kv_dtype, a->num_q_heads / a->num_kv_heads, cus)
                        : (short_units ? 2 * max_workers : max_workers);
    nw = (int)std::min<int64_t>(cap, std::max<int64_t>(1, (tiles_upper + kMinTilesPerWorker - 1) /
                                                              kMinTilesPerWorker));
    // a second wave on only some SIMDs leaves the others idle at the end: whole rounds only
    // (600 rows of 16 tokens: 1,200 workers 52.6 us, 1,024 46.3 us, 2,048 40.6 us)
    if (short_units && nw > max_workers) nw = 2 * max_workers;
  }
  plan->num_workers = nw;
  plan->tile_tokens = tile;
  if (decode_unit_mode(a, cus) && decode_unit_pieces(a, cus) > 1) {
    // few units: each cut over S workgroups (num_workers reports the S x units pieces),
    // whose partials take the split layout below with S x units slots past the units
    const size_t units = (size_t)a->num_seqs * a->num_kv_heads;
    const int S = decode_unit_pieces(a, cus);
    plan->num_workers = (int32_t)(units * S);
    const size_t slots = (units + units * S) * (size_t)(a->num_q_heads / a->num_kv_heads);
    plan->workspace_bytes = round_up(2 * units * sizeof(int32_t), 256) + 2 * round_up(slots * sizeof(float), 256) +
                            round_up(slots * kHeadDim * sizeof(float), 256);
  } else if (decode_unit_mode(a, cus)) {
    // one workgroup of 8 (or 4) waves per (row, kv head) unit, merged in LDS
    const int waves = unit_waves(a->kv_dtype, a->num_q_heads / a->num_kv_heads);
    plan->num_workers = (int32_t)std::min<int64_t>((int64_t)a->num_seqs * a->num_kv_heads * waves, INT32_MAX);
    plan->workspace_bytes = 0;
  } else if (a->num_seqs == 0) {
    plan->workspace_bytes = 0;
  } else {
    const size_t units = (size_t)a->num_seqs * a->num_kv_heads;
    const size_t slots = (units + nw) * (size_t)(a->num_q_heads / a->num_kv_heads);
    plan->workspace_bytes = round_up(2 * units * sizeof(int32_t), 256) + 2 * round_up(slots * sizeof(float), 256) +
                            round_up(slots * kHeadDim * sizeof(float), 256);
  }
  return PA_OK;
}

pa_status make_decode_launch(const pa_decode_args *a, const pa_plan &plan, DecodeLaunch *L) {
  std::memset(L, 0, sizeof *L);
  L->q = a->q;
  L->k_pool = a->k_pool;
  L->v_pool = a->v_pool;
  L->k_scale = a->k_scale;
  L->v_scale = a->v_scale;
  L->block_table = a->block_table;
  L->seq_lens = a->seq_lens;
  L->out = a->out;
  L->num_seqs = a->num_seqs;
  L->num_q_heads = a->num_q_heads;
  L->num_kv_heads = a->num_kv_heads;
  L->block_size = a->block_size;
  L->max_blocks_per_seq = a->max_blocks_per_seq;
  L->num_blocks = a->num_blocks;
  L->max_len = max_len_of(a);
  L->total_q = a->num_seqs;
  L->check_flags = device_check_flags();
  L->num_workers = plan.num_workers;
  L->workers_auto = a->num_workers == 0;
  L->min_tiles = kMinTilesPerWorker;
  L->unit_cost = kDecodeUnitCost;
  L->kv_dtype = a->kv_dtype;
  L->out_dtype = a->out_dtype;
  L->scale = a->scale;
  L->unit_mode = decode_unit_mode(a, device_cus());
  L->unit_pieces = L->unit_mode ? decode_unit_pieces(a, device_cus()) : 1;
  if (a->num_seqs > 0 && (!L->unit_mode || L->unit_pieces > 1)) {
    if (!a->workspace || a->workspace_bytes < plan.workspace_bytes)
      return set_error(PA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, plan needs %zu",
                       a->workspace ? a->workspace_bytes : (size_t)0, plan.workspace_bytes);
    const size_t units = (size_t)a->num_seqs * a->num_kv_heads;
    const size_t slots = (units + plan.num_workers) * (size_t)(a->num_q_heads / a->num_kv_heads);
    char *base = static_cast<char *>(a->workspace);
    L->seg_first = reinterpret_cast<int32_t *>(base);
    L->seg_count = L->seg_first + units;
    base += round_up(2 * units * sizeof(int32_t), 256);
    L->part_m = reinterpret_cast<float *>(base);
    base += round_up(slots * sizeof(float), 256);
    L->part_l = reinterpret_cast<float *>(base);
    base += round_up(slots * sizeof(float), 256);
    L->part_acc = reinterpret_cast<float *>(base);
  }
  return PA_OK;
}

pa_status plan_mixed(const pa_mixed_args *a, bool need_device_pointers, MixedPlan *mp) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  const pa_decode_args &b = a->base;
  pa_status s = validate_decode(&b, need_device_pointers);
  if (s != PA_OK) return s;
  const int B = b.num_seqs;
  const int nd = a->num_decode_rows;
  const int nv = a->num_verify_rows;
  if (nd < 0 || nv < 0 || (int64_t)nd + nv > B)
    return set_error(PA_ERR_BAD_SHAPE, "num_decode_rows=%d, num_verify_rows=%d do not fit num_seqs=%d", nd,
                     nv, B);
  const int n_pre = B - nd - nv;
  if (B > 0 && need_device_pointers && !a->q_start_loc)
    return set_error(PA_ERR_NULL_POINTER, "q_start_loc is required");
  if (B > 0 && a->total_q < B)
    return set_error(PA_ERR_BAD_SHAPE, "total_q=%d < num_seqs=%d", a->total_q, B);
  const int G = b.num_q_heads / b.num_kv_heads;
  if (nv > 0) {
    if (a->max_verify_q_len < 1 || (int64_t)a->max_verify_q_len * G > kVerifyMaxCols)
      return set_error(PA_ERR_UNSUPPORTED,
                       "max_verify_q_len=%d with group size %d: need 1 <= max_verify_q_len * group <= %d",
                       a->max_verify_q_len, G, kVerifyMaxCols);
    if (a->max_verify_q_len > b.max_seq_len)
      return set_error(PA_ERR_BAD_SHAPE, "max_verify_q_len=%d > max_seq_len=%d", a->max_verify_q_len,
                       b.max_seq_len);
    if (b.q_dtype != PA_BF16)
      return set_error(PA_ERR_UNSUPPORTED, "verify rows need bf16 q (and a bf16 or FP8 KV cache)");
  }
  if (n_pre > 0) {
    if (a->max_q_len < 1 || a->max_q_len > b.max_seq_len)
      return set_error(PA_ERR_BAD_SHAPE, "max_q_len=%d outside [1, max_seq_len=%d]", a->max_q_len,
                       b.max_seq_len);
    if (b.kv_dtype == PA_F32 || b.q_dtype != PA_BF16)
      return set_error(PA_ERR_UNSUPPORTED, "prefill-chunk rows need bf16 q and a bf16 or FP8 KV cache");
  }
  const int cus = device_cus();
  mp->cus = cus;
  pa_decode_args *dec = &mp->dec;
  pa_plan *dec_plan = &mp->dec_plan;
  int *verify_workers = &mp->verify_workers;
  size_t *verify_offset = &mp->verify_offset;
  *dec = b;
  dec->num_seqs = nd;
  plan_decode(dec, dec_plan);
  *verify_workers = 0;
  *verify_offset = round_up(dec_plan->workspace_bytes, 256);
  size_t vbytes = 0;
  if (nv > 0) {
    const int64_t units = (int64_t)nv * b.num_kv_heads;
    int nw = b.num_workers;
    if (nw == 0) {
      const int64_t tiles_upper = units * ((b.max_seq_len + kVerifyTile - 1) / kVerifyTile);
      nw = (int)std::min<int64_t>(mq_max_workers(b.kv_dtype, a->max_verify_q_len * G, cus),
                                  std::max<int64_t>(1, (tiles_upper + kMinTilesPerWorker - 1) / kMinTilesPerWorker));
    }
    *verify_workers = nw;
    const size_t slots = (size_t)(units + nw) * (size_t)(a->max_verify_q_len * G);
    vbytes = round_up(2 * (size_t)units * sizeof(int32_t), 256) + 2 * round_up(slots * sizeof(float), 256) +
             round_up(slots * kHeadDim * sizeof(float), 256);
  }
  size_t total = nv > 0 ? *verify_offset + vbytes : dec_plan->workspace_bytes;
  // prefill rows: a launch with at most half as many units as resident workgroups
  // cannot fill the chip, and its units can be long (a chunk after a long cached
  // prefix), so long units are cut into up to kPrefillMaxSplits kv pieces (of at
  // least kPrefillMinChunkTiles tiles) whose partials a merge kernel combines.  With
  // more units the pieces' extra traffic costs more than the balance gains (and in a
  // mixed batch the prefill already runs hidden beside the decode rows).
  mp->prefill_splits = 1;
  mp->prefill_waves = 4;
  mp->prefill_qtiles = 0;
  mp->prefill_offset = 0;
  mp->prefill_ml_offset = 0;
  mp->prefill_slots = 0;
  if (n_pre > 0) {
    const int hb = prefill_heads_per_block(G);
    auto units_of = [&](int waves) {
      const int qb = prefill_queries_per_block(G, waves);
      return (int64_t)n_pre * b.num_kv_heads * (G / hb) * ((a->max_q_len + qb - 1) / qb);
    };
    // prefill rows alone take the 8-wave shape when its units fill two or more rounds of its
    // resident workgroups (then the CUs stay balanced) or few enough to be cut into pieces;
    // otherwise, and beside decode or verify rows (whose kernel leaves room for the smaller
    // workgroups), the 4-wave shape
    const int64_t u8 = units_of(8);
    const int s8 = prefill_slots(cus, 8);
    const int waves = (n_pre == B && (u8 >= 2 * (int64_t)s8 || u8 <= s8 / 2)) ? 8 : 4;
    mp->prefill_waves = waves;
    const int qb = prefill_queries_per_block(G, waves);
    mp->prefill_qtiles = (a->max_q_len + qb - 1) / qb;
    const int64_t units_upper = units_of(waves);
    const int64_t tiles_upper = (b.max_seq_len + prefill_tile(waves) - 1) / prefill_tile(waves);
    int splits = 1;
    const int slots = prefill_slots(cus, waves);
    if (units_upper <= slots / 2) {
      splits = (int)std::min<int64_t>(kPrefillMaxSplits, (2 * slots + units_upper - 1) / units_upper);
      splits = (int)std::min<int64_t>(splits, std::max<int64_t>(1, tiles_upper / kPrefillMinChunkTiles));
    }
    mp->prefill_splits = splits;
    if (splits > 1) {
      mp->prefill_slots = (size_t)units_upper * splits;
      mp->prefill_offset = round_up(total, 256);
      mp->prefill_ml_offset =
          mp->prefill_offset + round_up(mp->prefill_slots * waves * 32 * kHeadDim * sizeof(float), 256);
      total = mp->prefill_ml_offset + round_up(mp->prefill_slots * waves * 32 * 2 * sizeof(float), 256);
    }
  }
  mp->total_bytes = total;
  return PA_OK;
}

pa_status make_verify_launch(const pa_mixed_args *a, int workers, size_t verify_offset, VerifyLaunch *V) {
  std::memset(V, 0, sizeof *V);
  const pa_decode_args &b = a->base;
  const int G = b.num_q_heads / b.num_kv_heads;
  V->q = b.q;
  V->k_pool = b.k_pool;
  V->v_pool = b.v_pool;
  V->block_table = b.block_table;
  V->seq_lens = b.seq_lens;
  V->q_start_loc = a->q_start_loc;
  V->out = b.out;
  V->k_scale = b.k_scale;
  V->v_scale = b.v_scale;
  V->item_kind = 0;
  V->kv_dtype = b.kv_dtype;
  V->first_row = a->num_decode_rows;
  V->num_rows = a->num_verify_rows;
  V->num_q_heads = b.num_q_heads;
  V->num_kv_heads = b.num_kv_heads;
  V->block_size = b.block_size;
  V->max_blocks_per_seq = b.max_blocks_per_seq;
  V->num_blocks = b.num_blocks;
  V->max_len = max_len_of(&b);
  V->total_q = a->total_q;
  V->check_flags = device_check_flags();
  V->num_workers = workers;
  V->workers_auto = b.num_workers == 0;
  V->min_tiles = kMinTilesPerWorker;
  V->slot_cols = a->max_verify_q_len * G;
  V->unit_cost = kMqUnitCost;
  V->out_dtype = b.out_dtype;
  V->scale = b.scale;
  const size_t units = (size_t)a->num_verify_rows * b.num_kv_heads;
  const size_t slots = (units + workers) * (size_t)V->slot_cols;
  char *base = static_cast<char *>(b.workspace) + verify_offset;
  V->seg_first = reinterpret_cast<int32_t *>(base);
  V->seg_count = V->seg_first + units;
  base += round_up(2 * units * sizeof(int32_t), 256);
  V->part_m = reinterpret_cast<float *>(base);
  base += round_up(slots * sizeof(float), 256);
  V->part_l = reinterpret_cast<float *>(base);
  base += round_up(slots * sizeof(float), 256);
  V->part_acc = reinterpret_cast<float *>(base);
  return PA_OK;
}

pa_status plan_cascade(const pa_cascade_args *a, bool need_device_pointers, DecodeLaunch *dec,
                       VerifyLaunch *pre, CascadeMergeLaunch *mrg, size_t *total_bytes) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  const pa_decode_args &b = a->base;
  pa_status s = validate_decode(&b, need_device_pointers);
  if (s != PA_OK) return s;
  if (b.num_seqs > 0 && (b.q_dtype != PA_BF16 || b.kv_dtype != PA_BF16))
    return set_error(PA_ERR_UNSUPPORTED, "shared-prefix decode needs bf16 q and a bf16 KV cache");
  const int B = b.num_seqs;
  const int G = b.num_q_heads / b.num_kv_heads;
  if (B > 0 && (a->num_groups < 1 || a->num_groups > B))
    return set_error(PA_ERR_BAD_SHAPE, "num_groups=%d outside [1, num_seqs=%d]", a->num_groups, B);
  if (B > 0 && (a->max_group_rows < 1 || (int64_t)a->max_group_rows * G > kVerifyMaxCols))
    return set_error(PA_ERR_UNSUPPORTED,
                     "max_group_rows=%d with group size %d: need 1 <= max_group_rows * group <= %d",
                     a->max_group_rows, G, kVerifyMaxCols);
  if (need_device_pointers && B > 0 && (!a->group_start || !a->shared_len))
    return set_error(PA_ERR_NULL_POINTER, "group_start and shared_len are required");
  // row parts: at most one worker per SIMD when the library chooses (their pieces all
  // become partials, so fewer, longer pieces pay off)
  pa_decode_args rows = b;
  if (rows.num_workers == 0) {
    pa_plan p0;
    plan_decode(&rows, &p0);
    rows.num_workers = std::min(p0.num_workers, verify_max_workers(device_cus()));
  }
  pa_plan dplan;
  plan_decode(&rows, &dplan);
  const size_t pre_offset = round_up(dplan.workspace_bytes, 256);
  size_t pbytes = 0;
  int pw = 0;
  const size_t punits = B > 0 ? (size_t)a->num_groups * b.num_kv_heads : 0;
  const int slot_cols = a->max_group_rows * G;
  if (B > 0) {
    pw = b.num_workers;
    if (pw == 0) {
      const int64_t tiles_upper = (int64_t)punits * ((b.max_seq_len + kVerifyTile - 1) / kVerifyTile);
      pw = (int)std::min<int64_t>(verify_max_workers(device_cus()),
                                  std::max<int64_t>(1, (tiles_upper + kMinTilesPerWorker - 1) / kMinTilesPerWorker));
    }
    const size_t slots = (punits + pw) * (size_t)slot_cols;
    pbytes = round_up(2 * punits * sizeof(int32_t), 256) + 2 * round_up(slots * sizeof(float), 256) +
             round_up(slots * kHeadDim * sizeof(float), 256);
  }
  *total_bytes = B > 0 ? pre_offset + pbytes : 0;
  if (!need_device_pointers || B == 0) return PA_OK;
  if (!b.workspace || b.workspace_bytes < *total_bytes)
    return set_error(PA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, the call needs %zu",
                     b.workspace ? b.workspace_bytes : (size_t)0, *total_bytes);
  s = make_decode_launch(&rows, dplan, dec);
  if (s != PA_OK) return s;
  dec->kv_start = a->shared_len;
  dec->workers_auto = b.num_workers == 0;
  dec->min_tiles = kCascadeRowMinTiles;
  // prefix kernel: items are the groups
  std::memset(pre, 0, sizeof *pre);
  pre->q = b.q;
  pre->k_pool = b.k_pool;
  pre->v_pool = b.v_pool;
  pre->block_table = b.block_table;
  pre->seq_lens = b.seq_lens;
  pre->group_start = a->group_start;
  pre->shared_len = a->shared_len;
  pre->item_kind = 1;
  pre->kv_dtype = PA_BF16;
  pre->num_rows = a->num_groups;
  pre->num_q_heads = b.num_q_heads;
  pre->num_kv_heads = b.num_kv_heads;
  pre->block_size = b.block_size;
  pre->max_blocks_per_seq = b.max_blocks_per_seq;
  pre->num_blocks = b.num_blocks;
  pre->max_len = max_len_of(&b);
  pre->total_q = b.num_seqs;
  pre->check_flags = device_check_flags();
  pre->num_workers = pw;
  pre->workers_auto = b.num_workers == 0;
  pre->min_tiles = kCascadePrefixMinTiles;
  pre->slot_cols = slot_cols;
  pre->unit_cost = kMqUnitCost;
  pre->out_dtype = b.out_dtype;
  pre->scale = b.scale;
  const size_t slots = (punits + pw) * (size_t)slot_cols;
  char *base = static_cast<char *>(b.workspace) + pre_offset;
  pre->seg_first = reinterpret_cast<int32_t *>(base);
  pre->seg_count = pre->seg_first + punits;
  base += round_up(2 * punits * sizeof(int32_t), 256);
  pre->part_m = reinterpret_cast<float *>(base);
  base += round_up(slots * sizeof(float), 256);
  pre->part_l = reinterpret_cast<float *>(base);
  base += round_up(slots * sizeof(float), 256);
  pre->part_acc = reinterpret_cast<float *>(base);
  // final merge
  std::memset(mrg, 0, sizeof *mrg);
  mrg->group_start = a->group_start;
  mrg->shared_len = a->shared_len;
  mrg->seg_first = dec->seg_first;
  mrg->seg_count = dec->seg_count;
  mrg->part_m = dec->part_m;
  mrg->part_l = dec->part_l;
  mrg->part_acc = dec->part_acc;
  mrg->pseg_first = pre->seg_first;
  mrg->pseg_count = pre->seg_count;
  mrg->ppart_m = pre->part_m;
  mrg->ppart_l = pre->part_l;
  mrg->ppart_acc = pre->part_acc;
  mrg->out = b.out;
  mrg->num_seqs = B;
  mrg->num_groups = a->num_groups;
  mrg->num_q_heads = b.num_q_heads;
  mrg->num_kv_heads = b.num_kv_heads;
  mrg->slot_cols = slot_cols;
  mrg->out_dtype = b.out_dtype;
  mrg->row_workers = dec->num_workers;
  mrg->prefix_workers = pw;
  return PA_OK;
}

pa_status make_decode_mq_launch(const pa_decode_args *a, const pa_plan &plan, VerifyLaunch *V) {
  DecodeLaunch L;
  pa_status s = make_decode_launch(a, plan, &L);
  if (s != PA_OK) return s;
  std::memset(V, 0, sizeof *V);
  V->q = a->q;
  V->k_pool = a->k_pool;
  V->v_pool = a->v_pool;
  V->block_table = a->block_table;
  V->seq_lens = a->seq_lens;
  V->out = a->out;
  V->seg_first = L.seg_first;
  V->seg_count = L.seg_count;
  V->part_m = L.part_m;
  V->part_l = L.part_l;
  V->part_acc = L.part_acc;
  V->k_scale = a->k_scale;
  V->v_scale = a->v_scale;
  V->item_kind = 2;
  V->kv_dtype = a->kv_dtype;
  V->first_row = 0;
  V->num_rows = a->num_seqs;
  V->num_q_heads = a->num_q_heads;
  V->num_kv_heads = a->num_kv_heads;
  V->block_size = a->block_size;
  V->max_blocks_per_seq = a->max_blocks_per_seq;
  V->num_blocks = a->num_blocks;
  V->max_len = max_len_of(a);
  V->total_q = a->num_seqs;
  V->check_flags = device_check_flags();
  V->num_workers = plan.num_workers;
  V->workers_auto = a->num_workers == 0;
  V->min_tiles = kMinTilesPerWorker;
  V->slot_cols = a->num_q_heads / a->num_kv_heads;
  V->unit_cost = kMqUnitCost;
  V->out_dtype = a->out_dtype;
  V->scale = a->scale;
  return PA_OK;
}

pa_status validate_append(const pa_append_args *a, bool need_device_pointers) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  if (a->num_tokens < 0) return set_error(PA_ERR_BAD_SHAPE, "num_tokens=%d < 0", a->num_tokens);
  if (a->num_kv_heads < 1) return set_error(PA_ERR_BAD_SHAPE, "num_kv_heads=%d < 1", a->num_kv_heads);
  if (a->head_dim != kHeadDim)
    return set_error(PA_ERR_UNSUPPORTED, "head_dim=%d (supported: %d)", a->head_dim, kHeadDim);
  if (!is_pow2_block(a->block_size))
    return set_error(PA_ERR_UNSUPPORTED, "block_size=%d (supported: 16, 32, 64, 128)", a->block_size);
  if (a->num_blocks < 1) return set_error(PA_ERR_BAD_SHAPE, "num_blocks=%d < 1", a->num_blocks);
  if ((int64_t)a->num_blocks * a->block_size > INT32_MAX)
    return set_error(PA_ERR_UNSUPPORTED, "num_blocks * block_size must fit in int32 slot numbers");
  const bool src_ok = a->src_dtype == PA_F32 || a->src_dtype == PA_BF16;
  const bool fp8 = a->kv_dtype == PA_FP8_E4M3;
  if (!src_ok || !(a->kv_dtype == a->src_dtype || fp8))
    return set_error(PA_ERR_BAD_DTYPE, "unsupported (src, kv) dtypes (%d, %d); supported: (f32, f32), "
                     "(bf16, bf16), (f32|bf16, fp8_e4m3)", a->src_dtype, a->kv_dtype);
  if (!fp8 && (a->k_scale || a->v_scale))
    return set_error(PA_ERR_BAD_DTYPE, "k_scale/v_scale are only used with an FP8 KV cache");
  if (need_device_pointers && a->num_tokens > 0) {
    if (!a->k || !a->v || !a->slot_mapping || !a->k_pool || !a->v_pool)
      return set_error(PA_ERR_NULL_POINTER, "k, v, slot_mapping, k_pool and v_pool are required");
    if (fp8 && (!a->k_scale || !a->v_scale))
      return set_error(PA_ERR_NULL_POINTER, "an FP8 KV cache needs k_scale and v_scale");
    if (!aligned16(a->k) || !aligned16(a->v) || !aligned16(a->k_pool) || !aligned16(a->v_pool))
      return set_error(PA_ERR_MISALIGNED, "k, v, k_pool and v_pool must be 16-byte aligned");
  }
  return PA_OK;
}

namespace {

pa_status check_rows(const pa_decode_args *a, const int32_t *qsl, int n_dec, int n_ver, int max_ver_q,
                     int max_q_len) {
  const int bs = a->block_size;
  for (int b = 0; b < a->num_seqs; ++b) {
    const int L = a->seq_lens[b];
    if (L < 1)
      return set_error(PA_ERR_BAD_METADATA, "seq_lens[%d]=%d < 1", b, L);
    if (L > a->max_seq_len)
      return set_error(PA_ERR_BAD_METADATA, "seq_lens[%d]=%d > max_seq_len=%d", b, L, a->max_seq_len);
    if ((int64_t)L > (int64_t)a->max_blocks_per_seq * bs)
      return set_error(PA_ERR_BAD_METADATA, "seq_lens[%d]=%d needs more than %d blocks", b, L,
                       a->max_blocks_per_seq);
    const int nb = (L + bs - 1) / bs;
    const int32_t *row = a->block_table + (size_t)b * a->max_blocks_per_seq;
    for (int j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= a->num_blocks)
        return set_error(PA_ERR_BAD_METADATA, "block_table[%d][%d]=%d outside [0, %d)", b, j, row[j],
                         a->num_blocks);
    if (qsl) {
      const int ql = qsl[b + 1] - qsl[b];
      if (ql < 1 || ql > L)
        return set_error(PA_ERR_BAD_METADATA, "row %d: q_len=%d outside [1, seq_len=%d]", b, ql, L);
      if (b < n_dec && (ql != 1 || qsl[b] != b))
        return set_error(PA_ERR_BAD_METADATA, "decode row %d must have q_len 1 at q index %d", b, b);
      if (b >= n_dec && b < n_dec + n_ver && ql > max_ver_q)
        return set_error(PA_ERR_BAD_METADATA, "verify row %d: q_len=%d > max_verify_q_len=%d", b, ql,
                         max_ver_q);
      if (b >= n_dec + n_ver && ql > max_q_len)
        return set_error(PA_ERR_BAD_METADATA, "row %d: q_len=%d > max_q_len=%d", b, ql, max_q_len);
    }
  }
  return PA_OK;
}

}  // namespace

pa_status check_append_decode_pair(const pa_append_args *app, const pa_decode_args *dec,
                                   bool need_device_pointers) {
  if (!app || !dec) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  pa_status s = validate_append(app, need_device_pointers);
  if (s != PA_OK) return s;
  s = validate_decode(dec, need_device_pointers);
  if (s != PA_OK) return s;
  if (app->num_tokens != dec->num_seqs)
    return set_error(PA_ERR_BAD_SHAPE, "num_tokens=%d != num_seqs=%d: one new token per decode row",
                     app->num_tokens, dec->num_seqs);
  if (app->k_pool != dec->k_pool || app->v_pool != dec->v_pool || app->kv_dtype != dec->kv_dtype ||
      app->num_kv_heads != dec->num_kv_heads || app->block_size != dec->block_size ||
      app->num_blocks != dec->num_blocks || app->k_scale != dec->k_scale || app->v_scale != dec->v_scale)
    return set_error(PA_ERR_BAD_SHAPE, "the append and decode arguments must describe the same pools");
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char *pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_POINTER: return "PA_ERR_NULL_POINTER";
    case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE";
    case PA_ERR_BAD_DTYPE: return "PA_ERR_BAD_DTYPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_MISALIGNED: return "PA_ERR_MISALIGNED";
    case PA_ERR_BAD_METADATA: return "PA_ERR_BAD_METADATA";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_decode_plan(const pa_decode_args *a, pa_plan *plan) {
  if (!plan) return set_error(PA_ERR_NULL_POINTER, "plan is NULL");
  pa_status s = validate_decode(a, false);
  if (s != PA_OK) return s;
  return plan_decode(a, plan);
}

size_t pa_decode_workspace_size(const pa_decode_args *a) {
  pa_plan plan;
  if (pa_decode_plan(a, &plan) != PA_OK) return SIZE_MAX;
  return plan.workspace_bytes;
}

pa_status pa_mixed_workspace_size(const pa_mixed_args *a, size_t *bytes) {
  if (!a || !bytes) return set_error(PA_ERR_NULL_POINTER, "argument is NULL");
  MixedPlan mp;
  pa_status s = plan_mixed(a, false, &mp);
  if (s == PA_OK) *bytes = mp.total_bytes;
  return s;
}

pa_status pa_check_decode_metadata(const pa_decode_args *a) {
  pa_status s = validate_decode(a, false);
  if (s != PA_OK) return s;
  if (a->num_seqs > 0 && (!a->seq_lens || !a->block_table))
    return set_error(PA_ERR_NULL_POINTER, "seq_lens and block_table host copies are required");
  return check_rows(a, nullptr, 0, 0, 0, 0);
}

pa_status pa_check_append_metadata(const pa_append_args *a) {
  pa_status s = validate_append(a, false);
  if (s != PA_OK) return s;
  if (a->num_tokens > 0 && !a->slot_mapping)
    return set_error(PA_ERR_NULL_POINTER, "slot_mapping host copy is required");
  const int64_t nslots = (int64_t)a->num_blocks * a->block_size;
  std::vector<char> used((size_t)nslots, 0);
  for (int t = 0; t < a->num_tokens; ++t) {
    const int32_t sl = a->slot_mapping[t];
    if (sl < -1 || sl >= nslots)
      return set_error(PA_ERR_BAD_METADATA, "slot_mapping[%d]=%d outside [-1, %lld)", t, sl, (long long)nslots);
    if (sl >= 0) {
      if (used[(size_t)sl]) return set_error(PA_ERR_BAD_METADATA, "slot %d written by two tokens", sl);
      used[(size_t)sl] = 1;
    }
  }
  return PA_OK;
}

pa_status pa_check_append_decode_metadata(const pa_append_args *app, const pa_decode_args *dec) {
  pa_status s = check_append_decode_pair(app, dec, false);
  if (s != PA_OK) return s;
  s = pa_check_append_metadata(app);
  if (s != PA_OK) return s;
  s = pa_check_decode_metadata(dec);
  if (s != PA_OK) return s;
  // token b is row b's newest position
  for (int b = 0; b < dec->num_seqs; ++b) {
    const int32_t slot = app->slot_mapping[b];
    if (slot < 0) continue;
    const int pos = dec->seq_lens[b] - 1;
    const int64_t want = (int64_t)dec->block_table[(size_t)b * dec->max_blocks_per_seq + pos / dec->block_size] *
                             dec->block_size + pos % dec->block_size;
    if (slot != want)
      return set_error(PA_ERR_BAD_METADATA, "slot_mapping[%d]=%d is not the slot of row %d's position %d (%lld)",
                       b, slot, b, pos, (long long)want);
  }
  return PA_OK;
}

pa_status pa_check_mixed_metadata(const pa_mixed_args *a) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  MixedPlan mp;
  pa_status s = plan_mixed(a, false, &mp);
  if (s != PA_OK) return s;
  const int B = a->base.num_seqs;
  if (B > 0 && (!a->base.seq_lens || !a->base.block_table || !a->q_start_loc))
    return set_error(PA_ERR_NULL_POINTER, "seq_lens, block_table and q_start_loc host copies are required");
  if (B > 0) {
    if (a->q_start_loc[0] != 0)
      return set_error(PA_ERR_BAD_METADATA, "q_start_loc[0]=%d != 0", a->q_start_loc[0]);
    if (a->q_start_loc[B] != a->total_q)
      return set_error(PA_ERR_BAD_METADATA, "q_start_loc[%d]=%d != total_q=%d", B, a->q_start_loc[B],
                       a->total_q);
  }
  return check_rows(&a->base, a->q_start_loc, a->num_decode_rows, a->num_verify_rows, a->max_verify_q_len,
                    a->max_q_len);
}

pa_status pa_check_metadata(const pa_mixed_args *a) { return pa_check_mixed_metadata(a); }

pa_status pa_cascade_workspace_size(const pa_cascade_args *a, size_t *bytes) {
  if (!a || !bytes) return set_error(PA_ERR_NULL_POINTER, "argument is NULL");
  DecodeLaunch d;
  VerifyLaunch v;
  CascadeMergeLaunch m;
  return plan_cascade(a, false, &d, &v, &m, bytes);
}

pa_status pa_check_cascade_metadata(const pa_cascade_args *a) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  DecodeLaunch d;
  VerifyLaunch v;
  CascadeMergeLaunch m;
  size_t total = 0;
  pa_status s = plan_cascade(a, false, &d, &v, &m, &total);
  if (s != PA_OK) return s;
  const pa_decode_args &b = a->base;
  const int B = b.num_seqs;
  if (B == 0) return PA_OK;
  if (!b.seq_lens || !b.block_table || !a->group_start || !a->shared_len)
    return set_error(PA_ERR_NULL_POINTER, "seq_lens, block_table, group_start and shared_len host copies are required");
  s = check_rows(&b, nullptr, 0, 0, 0, 0);
  if (s != PA_OK) return s;
  const int32_t *gs = a->group_start;
  if (gs[0] != 0 || gs[a->num_groups] != B)
    return set_error(PA_ERR_BAD_METADATA, "group_start must run from 0 to num_seqs=%d (got %d .. %d)", B, gs[0],
                     gs[a->num_groups]);
  const int bs = b.block_size;
  for (int k = 0; k < a->num_groups; ++k) {
    const int r0 = gs[k], r1 = gs[k + 1];
    if (r1 <= r0) return set_error(PA_ERR_BAD_METADATA, "group %d is empty (group_start not increasing)", k);
    if (r1 - r0 > a->max_group_rows)
      return set_error(PA_ERR_BAD_METADATA, "group %d has %d rows > max_group_rows=%d", k, r1 - r0,
                       a->max_group_rows);
    const int P = a->shared_len[r0];
    const int32_t *t0 = b.block_table + (size_t)r0 * b.max_blocks_per_seq;
    for (int r = r0; r < r1; ++r) {
      if (a->shared_len[r] != P)
        return set_error(PA_ERR_BAD_METADATA, "row %d: shared_len=%d differs from its group's %d", r,
                         a->shared_len[r], P);
      if (P < 0 || P % bs != 0 || P >= b.seq_lens[r])
        return set_error(PA_ERR_BAD_METADATA,
                         "row %d: shared_len=%d must be a multiple of block_size=%d below seq_len=%d", r, P, bs,
                         b.seq_lens[r]);
      const int32_t *tr = b.block_table + (size_t)r * b.max_blocks_per_seq;
      for (int j = 0; j < P / bs; ++j)
        if (tr[j] != t0[j])
          return set_error(PA_ERR_BAD_METADATA, "row %d: block %d of the shared prefix is %d, its group's is %d", r,
                           j, tr[j], t0[j]);
    }
  }
  return PA_OK;
}

}  // extern "C"
