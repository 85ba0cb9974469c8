/*
 * pa_runtime.h -- host-side C ABI of the paged KV cache manager and scheduler.
 *
 * What it models:
 *   - a pool of equal blocks, a per-request list of blocks that grows by one
 *     block when the last one is full, blocks returned to the pool when a
 *     request finishes ("How does TensorRT-LLM work" (outcomeschool.com),
 *     section "The paged KV cache"; "TensorRT-LLM, in depth"
 *     (aicassindra.com), section "The paged KV cache and block reuse");
 *   - prefix reuse: requests whose prompts begin with the same whole blocks of
 *     tokens point at the same physical blocks (same sections);
 *   - one scheduler iteration of in-flight batching: requests that are
 *     decoding take one token each, in admission order, while the batch has
 *     room and the token budget lasts; a decoding request that needs a new
 *     block and finds none is skipped this iteration; then waiting requests
 *     take prefill chunks (what is left of the prompt after reused blocks and
 *     earlier chunks, cut to the remaining budget), admission stopping at the
 *     first that cannot get its blocks ("TensorRT-LLM, in depth", section
 *     "In-flight batching and the scheduler").  Decode rows come first in the
 *     batch, as pa_mixed expects.
 *
 * Pure host code: no HIP calls, no device memory.  The batch it produces is
 * the metadata of one pass (block table, seq_lens, q_start_loc, slot mapping)
 * in host memory owned by the manager; the caller copies it to the device and
 * launches pa_append and pa_mixed (or pa_decode) with it.
 *
 * Ownership and errors: a manager is created and destroyed by the caller;
 * batch arrays stay valid until the next pa_kvm_schedule or
 * pa_kvm_destroy on the same manager.  Calls return pa_status (pa.h);
 * pa_last_error() describes a non-OK status.  Not thread-safe: one manager is
 * used by one thread at a time.
 */
#ifndef PA_RUNTIME_H_
#define PA_RUNTIME_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_kvm pa_kvm;   /* opaque manager */

/* One pass's metadata (host arrays owned by the manager). */
typedef struct pa_kvm_batch {
  int32_t num_rows;            /* B requests in the pass */
  int32_t num_decode_rows;     /* rows [0, num_decode_rows) decode one token each */
  int32_t total_q;             /* new tokens in the pass */
  int32_t max_q_len;           /* largest q_len among the prefill rows (0 if none) */
  int32_t max_seq_len;         /* largest seq_len of the pass */
  int32_t max_blocks_per_seq;  /* row stride of block_table (fixed at creation) */
  const int64_t *request_ids;  /* [B] */
  const int32_t *seq_lens;     /* [B] cached tokens after this pass's tokens are appended */
  const int32_t *q_start_loc;  /* [B + 1] exclusive prefix sum of q_len */
  const int32_t *block_table;  /* [B][max_blocks_per_seq], -1 past a row's blocks */
  const int32_t *slot_mapping; /* [total_q] block * block_size + offset of each new token */
  const int32_t *positions;    /* [total_q] position of each new token in its request */
  const int32_t *token_ids;    /* [total_q] token id of each new token */
} pa_kvm_batch;

/* Read-only view of one request. */
typedef struct pa_kvm_request_info {
  int32_t state;               /* 0 waiting, 1 prefilling (some chunks done), 2 decoding, 3 finished */
  int32_t prompt_len;
  int32_t num_cached;          /* tokens whose K/V are in the cache */
  int32_t num_reused;          /* prompt tokens found in reused blocks at admission */
  int32_t num_generated;       /* tokens produced so far */
  int32_t num_blocks;          /* blocks held */
} pa_kvm_request_info;

/* num_blocks blocks of block_size tokens; a request may hold at most
 * max_blocks_per_seq blocks; prefix_reuse != 0 enables block reuse. */
pa_status pa_kvm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t prefix_reuse, pa_kvm **out);
void pa_kvm_destroy(pa_kvm *m);

/* Queue a request (ids unique).  It produces max_new_tokens >= 1 tokens, the
 * first at the end of its prompt's prefill.  prompt_len + max_new_tokens - 1
 * must fit in max_blocks_per_seq blocks. */
pa_status pa_kvm_add_request(pa_kvm *m, int64_t id, const int32_t *prompt, int32_t prompt_len,
                             int32_t max_new_tokens);

/* One scheduler iteration; fills *batch (possibly with zero rows). */
pa_status pa_kvm_schedule(pa_kvm *m, int32_t max_batch_size, int32_t max_num_tokens, pa_kvm_batch *batch);

/* After the pass: every row's tokens are now cached.  sampled[i] is the token
 * row i produced (read for decode rows and for prefill rows whose prompt is
 * complete; ignored otherwise).  Requests that reach max_new_tokens finish and
 * release their blocks. */
pa_status pa_kvm_complete(pa_kvm *m, const int32_t *sampled);

int32_t pa_kvm_num_free_blocks(const pa_kvm *m);
/* Blocks whose reference count is above zero (held by some request). */
int32_t pa_kvm_num_used_blocks(const pa_kvm *m);
pa_status pa_kvm_request_info_get(const pa_kvm *m, int64_t id, pa_kvm_request_info *info);
/* Tokens generated by a request so far (up to `cap` copied); returns the count via *n. */
pa_status pa_kvm_generated(const pa_kvm *m, int64_t id, int32_t *tokens, int32_t cap, int32_t *n);

#ifdef __cplusplus
}
#endif

#endif /* PA_RUNTIME_H_ */
