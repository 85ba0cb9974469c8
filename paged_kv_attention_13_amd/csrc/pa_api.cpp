// ABI entry points that queue work: validate on the host, then hand the
// resolved launch description to the kernel launchers.  Plain C++.
#include "pa_internal.h"

using namespace pa;

namespace {

pa_status prepare_decode(const pa_decode_args *a, pa_plan *plan, DecodeLaunch *L) {
  pa_status s = validate_decode(a, true);
  if (s != PA_OK) return s;
  plan_decode(a, plan);
  return make_decode_launch(a, *plan, L);
}

pa_status hip_status(int err, const char *what) {
  if (err == 0) return PA_OK;
  return set_error(PA_ERR_HIP, "%s launch failed: %s (%d)", what, hip_error_name(err), err);
}

}  // namespace

extern "C" {

pa_status pa_decode_partials(const pa_decode_args *a, void *stream) {
  pa_plan plan;
  DecodeLaunch L;
  pa_status s = prepare_decode(a, &plan, &L);
  if (s != PA_OK || a->num_seqs == 0) return s;
  return hip_status(launch_decode_partials(L, stream), "decode");
}

pa_status pa_merge_partials(const pa_decode_args *a, void *stream) {
  pa_plan plan;
  DecodeLaunch L;
  pa_status s = prepare_decode(a, &plan, &L);
  if (s != PA_OK || a->num_seqs == 0) return s;
  return hip_status(launch_merge(L, stream), "merge");
}

pa_status pa_decode(const pa_decode_args *a, void *stream) {
  pa_plan plan;
  DecodeLaunch L;
  pa_status s = prepare_decode(a, &plan, &L);
  if (s != PA_OK || a->num_seqs == 0) return s;
  s = hip_status(launch_decode_partials(L, stream), "decode");
  if (s != PA_OK) return s;
  return hip_status(launch_merge(L, stream), "merge");
}

pa_status pa_append(const pa_append_args *a, void *stream) {
  pa_status s = validate_append(a, true);
  if (s != PA_OK || a->num_tokens == 0) return s;
  AppendLaunch L{};
  L.k = a->k;
  L.v = a->v;
  L.slot_mapping = a->slot_mapping;
  L.k_pool = a->k_pool;
  L.v_pool = a->v_pool;
  L.k_scale = a->k_scale;
  L.v_scale = a->v_scale;
  L.num_tokens = a->num_tokens;
  L.num_kv_heads = a->num_kv_heads;
  L.block_size = a->block_size;
  L.src_dtype = a->src_dtype;
  L.kv_dtype = a->kv_dtype;
  return hip_status(launch_append(L, stream), "append");
}

pa_status pa_mixed(const pa_mixed_args *a, void *stream) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  const pa_decode_args &b = a->base;
  pa_status s = validate_decode(&b, true);
  if (s != PA_OK) return s;
  if (a->num_decode_rows < 0 || a->num_decode_rows > b.num_seqs)
    return set_error(PA_ERR_BAD_SHAPE, "num_decode_rows=%d outside [0, num_seqs=%d]",
                     a->num_decode_rows, b.num_seqs);
  const int n_pre = b.num_seqs - a->num_decode_rows;
  if (b.num_seqs > 0 && !a->q_start_loc)
    return set_error(PA_ERR_NULL_POINTER, "q_start_loc is required");
  if (a->total_q < b.num_seqs)
    return set_error(PA_ERR_BAD_SHAPE, "total_q=%d < num_seqs=%d", a->total_q, b.num_seqs);
  if (n_pre > 0) {
    if (a->max_q_len < 1 || a->max_q_len > b.max_seq_len)
      return set_error(PA_ERR_BAD_SHAPE, "max_q_len=%d outside [1, max_seq_len=%d]", a->max_q_len,
                       b.max_seq_len);
    if (b.kv_dtype != PA_BF16)
      return set_error(PA_ERR_UNSUPPORTED, "prefill-chunk rows need a bf16 KV cache and bf16 q");
  }
  // decode rows: a decode call over rows [0, num_decode_rows), whose q and out
  // rows are the first num_decode_rows rows of the packed q/out.
  pa_decode_args d = b;
  d.num_seqs = a->num_decode_rows;
  pa_plan plan;
  DecodeLaunch L;
  plan_decode(&d, &plan);
  if (d.num_seqs > 0) {
    s = make_decode_launch(&d, plan, &L);
    if (s != PA_OK) return s;
  }
  // validation is complete: queue the work
  if (n_pre > 0) {
    PrefillLaunch P{};
    P.q = b.q;
    P.k_pool = b.k_pool;
    P.v_pool = b.v_pool;
    P.block_table = b.block_table;
    P.seq_lens = b.seq_lens;
    P.q_start_loc = a->q_start_loc;
    P.out = b.out;
    P.first_row = a->num_decode_rows;
    P.num_rows = n_pre;
    P.num_q_heads = b.num_q_heads;
    P.num_kv_heads = b.num_kv_heads;
    P.block_size = b.block_size;
    P.max_blocks_per_seq = b.max_blocks_per_seq;
    P.max_q_len = a->max_q_len;
    P.out_dtype = b.out_dtype;
    P.scale = b.scale;
    s = hip_status(launch_prefill(P, stream), "prefill");
    if (s != PA_OK) return s;
  }
  if (d.num_seqs > 0) {
    s = hip_status(launch_decode_partials(L, stream), "decode");
    if (s != PA_OK) return s;
    return hip_status(launch_merge(L, stream), "merge");
  }
  return PA_OK;
}

}  // extern "C"
