// ABI entry points that queue work: validate on the host, then hand the
// resolved launch description to the kernel launchers.  Plain C++.
#include "pa_internal.h"
#include "pa_probe.h"

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
  if (decode_on_mq(a)) {
    VerifyLaunch V;
    s = make_decode_mq_launch(a, plan, &V);
    if (s != PA_OK) return s;
    return hip_status(launch_verify_partials(V, stream), "decode");
  }
  return hip_status(launch_decode_partials(L, stream), "decode");
}

int pa_device_checks(void) { return PA_DEVICE_CHECKS; }

pa_status pa_device_check_flags(uint32_t *flags) {
  if (!flags) return set_error(PA_ERR_NULL_POINTER, "flags is NULL");
  return hip_status(read_and_clear_check_flags(flags), "device check flags");
}

pa_status pa_decode_noalloc(const pa_decode_args *a, void *stream) {
  if (!a) return set_error(PA_ERR_NULL_POINTER, "argument struct is NULL");
  pa_decode_args b = *a;
  b.workspace = nullptr;                   // the caller's workspace fields are ignored
  b.workspace_bytes = 0;
  pa_status s = validate_decode(&b, true);
  if (s != PA_OK) return s;
  pa_plan plan;
  plan_decode(&b, &plan);
  if (plan.workspace_bytes > kStaticScratchBytes)
    return set_error(PA_ERR_WORKSPACE_TOO_SMALL,
                     "the call needs %zu bytes of split partials; the library's static scratch holds %zu "
                     "(pass a workspace to pa_decode instead)",
                     plan.workspace_bytes, kStaticScratchBytes);
  if (b.num_seqs > 0 && plan.workspace_bytes > 0) {
    // nothing in the scratch has to start at zero: the decode kernels write every unit's
    // piece record and every partial that the merge reads in the same call
    void *ptr = nullptr;
    s = hip_status(static_scratch(&ptr), "static scratch address");
    if (s != PA_OK) return s;
    b.workspace = ptr;
    b.workspace_bytes = kStaticScratchBytes;
  }
  return pa_decode(&b, stream);
}

pa_status pa_merge_partials(const pa_decode_args *a, void *stream) {
  pa_plan plan;
  DecodeLaunch L;
  pa_status s = prepare_decode(a, &plan, &L);
  if (s != PA_OK || a->num_seqs == 0) return s;
  if (decode_on_mq(a)) {
    VerifyLaunch V;
    s = make_decode_mq_launch(a, plan, &V);
    if (s != PA_OK) return s;
    return hip_status(launch_verify_merge(V, stream), "merge");
  }
  return hip_status(launch_merge(L, stream), "merge");
}

pa_status pa_decode(const pa_decode_args *a, void *stream) {
  pa_status s = pa_decode_partials(a, stream);
  if (s != PA_OK || !a || a->num_seqs == 0) return s;
  return pa_merge_partials(a, stream);
}

pa_status pa_append_decode(const pa_append_args *app, const pa_decode_args *dec, void *stream) {
  pa_status s = check_append_decode_pair(app, dec, true);
  if (s != PA_OK || dec->num_seqs == 0) return s;
  pa_plan plan;
  DecodeLaunch L;
  s = prepare_decode(dec, &plan, &L);
  if (s != PA_OK) return s;
  if (L.unit_mode) {
    // one launch (plus the merge when units are cut over several workgroups): the unit's
    // first workgroup appends its row's new token, and every workgroup takes position
    // seq_len - 1 from the new rows, so the results are those of pa_append + pa_decode
    L.k_new = app->k;
    L.v_new = app->v;
    L.new_slots = app->slot_mapping;
    L.k_pool_w = app->k_pool;
    L.v_pool_w = app->v_pool;
    s = hip_status(launch_decode_partials(L, stream), "append + decode");
    if (s != PA_OK) return s;
    return hip_status(launch_merge(L, stream), "merge");
  }
  s = pa_append(app, stream);
  if (s != PA_OK) return s;
  return pa_decode(dec, stream);
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
  L.num_blocks = a->num_blocks;
  L.check_flags = device_check_flags();
  return hip_status(launch_append(L, stream), "append");
}

pa_status pa_mixed(const pa_mixed_args *a, void *stream) {
  MixedPlan mp;
  pa_status s = plan_mixed(a, true, &mp);
  if (s != PA_OK) return s;
  const pa_decode_args &d = mp.dec;
  const pa_plan &plan = mp.dec_plan;
  const size_t total = mp.total_bytes;
  const pa_decode_args &b = a->base;
  if (total > 0 && (!b.workspace || b.workspace_bytes < total))
    return set_error(PA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, the batch needs %zu",
                     b.workspace ? b.workspace_bytes : (size_t)0, total);
  const int n_ver = a->num_verify_rows;
  const int n_pre = b.num_seqs - a->num_decode_rows - n_ver;
  // decode rows: a decode call over rows [0, num_decode_rows), whose q and out
  // rows are the first num_decode_rows rows of the packed q/out.
  DecodeLaunch L;
  if (d.num_seqs > 0) {
    s = make_decode_launch(&d, plan, &L);
    if (s != PA_OK) return s;
  }
  VerifyLaunch V;
  if (n_ver > 0) make_verify_launch(a, mp.verify_workers, mp.verify_offset, &V);
  // validation is complete: queue the work.  Prefill-chunk rows (matrix-core bound) run
  // on the auxiliary stream beside the decode and verify rows (HBM bound); the decode
  // kernel is queued first so that it takes its waves before the prefill workgroups.
  void *pre_stream = stream;
  const bool fork = n_pre > 0 && (d.num_seqs > 0 || n_ver > 0);
  if (fork) {
    s = hip_status(fork_side_stream(stream, &pre_stream), "stream fork");
    if (s != PA_OK) return s;
  }
  pa_status rs = PA_OK;
  if (d.num_seqs > 0) {
    if (decode_on_mq(&d)) {
      VerifyLaunch DV;
      rs = make_decode_mq_launch(&d, plan, &DV);
      if (rs == PA_OK) rs = hip_status(launch_verify_partials(DV, stream), "decode");
      if (rs == PA_OK) rs = hip_status(launch_verify_merge(DV, stream), "merge");
    } else {
      rs = hip_status(launch_decode_partials(L, stream), "decode");
      if (rs == PA_OK) rs = hip_status(launch_merge(L, stream), "merge");
    }
  }
  if (rs == PA_OK && n_ver > 0) {
    rs = hip_status(launch_verify_partials(V, stream), "verify");
    if (rs == PA_OK) rs = hip_status(launch_verify_merge(V, stream), "verify merge");
  }
  if (rs == PA_OK && n_pre > 0) {
    PrefillLaunch P{};
    P.q = b.q;
    P.k_pool = b.k_pool;
    P.v_pool = b.v_pool;
    P.k_scale = b.k_scale;
    P.v_scale = b.v_scale;
    P.kv_dtype = b.kv_dtype;
    P.block_table = b.block_table;
    P.seq_lens = b.seq_lens;
    P.q_start_loc = a->q_start_loc;
    P.out = b.out;
    P.first_row = a->num_decode_rows + n_ver;
    P.num_rows = n_pre;
    P.num_q_heads = b.num_q_heads;
    P.num_kv_heads = b.num_kv_heads;
    P.block_size = b.block_size;
    P.max_blocks_per_seq = b.max_blocks_per_seq;
    P.num_blocks = b.num_blocks;
    P.max_len = max_len_of(&b);
    P.total_q = a->total_q;
    P.check_flags = device_check_flags();
    P.max_q_len = a->max_q_len;
    P.out_dtype = b.out_dtype;
    P.scale = b.scale;
    P.splits = mp.prefill_splits;
    P.max_qtiles = mp.prefill_qtiles;
    P.resident_slots = prefill_slots(mp.cus, mp.prefill_waves);
    P.waves = mp.prefill_waves;
    if (mp.prefill_splits > 1) {
      char *ws = static_cast<char *>(b.workspace);
      P.part_o = reinterpret_cast<float *>(ws + mp.prefill_offset);
      P.part_ml = reinterpret_cast<float *>(ws + mp.prefill_ml_offset);
    }
    rs = hip_status(launch_prefill(P, pre_stream), "prefill");
    if (rs == PA_OK && mp.prefill_splits > 1) rs = hip_status(launch_prefill_merge(P, pre_stream), "prefill merge");
  }
  if (fork) {
    const pa_status js = hip_status(join_side_stream(stream), "stream join");
    if (rs == PA_OK) rs = js;
  }
  return rs;
}

pa_status pa_decode_cascade(const pa_cascade_args *a, void *stream) {
  DecodeLaunch d;
  VerifyLaunch pre;
  CascadeMergeLaunch m;
  size_t total = 0;
  pa_status s = plan_cascade(a, true, &d, &pre, &m, &total);
  if (s != PA_OK || a->base.num_seqs == 0) return s;
  s = hip_status(launch_verify_partials(pre, stream), "shared-prefix");
  if (s != PA_OK) return s;
  s = hip_status(launch_decode_partials(d, stream), "decode");
  if (s != PA_OK) return s;
  return hip_status(launch_cascade_merge(m, stream), "cascade merge");
}

pa_status pa_stream_read(const void *src, size_t bytes, uint32_t *out, int32_t num_workgroups,
                         int32_t loads_in_flight, void *stream) {
  if (!src || !out) return set_error(PA_ERR_NULL_POINTER, "src and out are required");
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return set_error(PA_ERR_MISALIGNED, "src must be 16-byte aligned and out 4-byte aligned");
  if (bytes == 0 || bytes % 16 != 0)
    return set_error(PA_ERR_BAD_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
  if (num_workgroups < 1 || num_workgroups > 65536)
    return set_error(PA_ERR_BAD_SHAPE, "num_workgroups=%d outside [1, 65536]", num_workgroups);
  if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16)
    return set_error(PA_ERR_UNSUPPORTED, "loads_in_flight=%d (supported: 4, 8, 16)", loads_in_flight);
  return hip_status(launch_stream_read(src, bytes, out, num_workgroups, loads_in_flight, stream), "stream read");
}

pa_status pa_gather_read(const void *base, const int64_t *page_offsets, int64_t num_pages, int32_t page_bytes,
                         uint32_t *out, int32_t num_workgroups, int32_t pages_in_flight, void *stream) {
  if (!base || !page_offsets || !out) return set_error(PA_ERR_NULL_POINTER, "base, page_offsets and out are required");
  if ((reinterpret_cast<uintptr_t>(base) & 15u) != 0 || (reinterpret_cast<uintptr_t>(page_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return set_error(PA_ERR_MISALIGNED, "base must be 16-byte, page_offsets 8-byte and out 4-byte aligned");
  if (num_pages < 1 || page_bytes < 1024 || page_bytes % 1024 != 0)
    return set_error(PA_ERR_BAD_SHAPE, "num_pages=%lld must be >= 1 and page_bytes=%d a positive multiple of 1024",
                     (long long)num_pages, page_bytes);
  if (num_workgroups < 1 || num_workgroups > 65536)
    return set_error(PA_ERR_BAD_SHAPE, "num_workgroups=%d outside [1, 65536]", num_workgroups);
  if (pages_in_flight != 2 && pages_in_flight != 4 && pages_in_flight != 8)
    return set_error(PA_ERR_UNSUPPORTED, "pages_in_flight=%d (supported: 2, 4, 8)", pages_in_flight);
  return hip_status(launch_gather_read(base, page_offsets, num_pages, page_bytes, out, num_workgroups,
                                       pages_in_flight, stream),
                    "gather read");
}

}  // extern "C"
