/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-KV attention library.
 *
 * The library computes softmax attention of new query tokens against a KV
 * cache kept in a pool of equal fixed-size blocks, each request reaching its
 * tokens through an ordered block table:
 *   - the pool of equal blocks handed out on demand, and the small table that
 *     records which blocks belong to which request and in what order:
 *     "How does TensorRT-LLM work" (outcomeschool.com), section
 *     "The paged KV cache";
 *   - virtual-to-physical block tables over non-contiguous blocks:
 *     "Introduction to TensorRT-LLM" (dileepadev.github.io), section
 *     "2. Paged KV Cache";
 *   - each decode step reads the request's entire KV cache and is therefore
 *     memory-bandwidth-bound; grouped-query attention with 8 KV heads for
 *     Llama-3-8B: "TensorRT-LLM, in depth" (aicassindra.com), section
 *     "First principles: where the GPU memory goes";
 *   - prefill chunks mixed with decode rows in one pass: same page, section
 *     "In-flight batching and the scheduler";
 *   - an FP8 KV cache: same page, section "Quantization: fewer bytes per
 *     weight and per cached token";
 *   - rows that check a few drafted tokens in one pass (speculative
 *     decoding): same page and "How does TensorRT-LLM work", sections
 *     "Speculative decoding".
 *
 * Operation (one layer).  For row b with L = seq_lens[b] cached tokens
 * (including the row's n new ones), new query i in [0, n), and query head h
 * of kv head g = h / (Hq / Hkv):
 *     K[t] = k_pool[block_table[b][t / bs]][g][t % bs][:]      (t < L)
 *     out[i][h] = sum_t softmax_t(scale * <q[i][h], K[t]>) V[t],
 *                 over t <= L - n + i (every earlier token and its own).
 * FP8 pools hold OCP E4M3 codes; the value is code * k_scale[g] (V: v_scale[g]).
 *
 * Memory layout (all row-major, densely packed, element strides implied):
 *     q, out       [rows][Hq][D]            rows = num_seqs (decode) or total_q
 *     k_pool,v_pool[num_blocks][Hkv][bs][D] one (block, kv head) page contiguous
 *     block_table  [num_seqs][max_blocks_per_seq] int32
 *     seq_lens     [num_seqs] int32
 *     q_start_loc  [num_seqs + 1] int32, exclusive prefix sum of q_len
 *
 * Pointers in the argument structs are DEVICE pointers except in the
 * pa_check_*_metadata calls, which read HOST copies.  The caller owns every
 * buffer, including the workspace (size from pa_decode_plan /
 * pa_mixed_workspace_size).  The library keeps no pointer after a call
 * returns, allocates no memory, and never synchronises: work is queued on
 * `stream` (a hipStream_t; NULL = the default stream) and the call returns.
 * pa_mixed runs a batch's prefill-chunk rows on an auxiliary stream beside
 * its decode and verify rows (event fork and join with `stream`, so all of
 * the call's work is ordered on `stream` as if queued there); that stream and
 * two events are created once per device, on first use.  Calls are safe to
 * record into a HIP graph.
 *
 * Errors.  Every host-checkable problem returns a status before anything is
 * launched: null pointers, misalignment (16 bytes for q, pools, out,
 * workspace), dtype combinations, Hq % Hkv, supported head_dim / block size /
 * group size, workspace too small, row classes that do not fit num_seqs.  Launch
 * failures return PA_ERR_HIP.  The device-resident metadata is a
 * PRECONDITION that the kernels do not re-check:
 *     1 <= q_len_b <= L_b <= max_seq_len <= max_blocks_per_seq * bs,
 *     q_len_b within its class's bound (1, max_verify_q_len, max_q_len),
 *     0 <= block_table[b][j] < num_blocks for j < ceil(L_b / bs).
 * pa_check_decode_metadata / pa_check_mixed_metadata verify it on host copies.
 * Table entries at j >= ceil(L_b / bs), pool slots past L_b in a row's last
 * block and blocks no row references are never read into the result.
 * No C++ exception crosses this interface.  pa_last_error() returns a
 * thread-local message describing the last non-OK status.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 4

/* Element types.  Supported (q, kv, out) combinations:
 *   (F32, F32, F32|BF16), (BF16, BF16, BF16|F32), (BF16, FP8_E4M3, BF16|F32). */
typedef enum {
  PA_F32 = 0,
  PA_BF16 = 1,
  PA_FP8_E4M3 = 2
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,
  PA_ERR_BAD_SHAPE = 2,
  PA_ERR_BAD_DTYPE = 3,
  PA_ERR_UNSUPPORTED = 4,
  PA_ERR_WORKSPACE_TOO_SMALL = 5,
  PA_ERR_MISALIGNED = 6,
  PA_ERR_BAD_METADATA = 7,
  PA_ERR_HIP = 8
} pa_status;

/* Arguments of a decode call: one new query token per row. */
typedef struct pa_decode_args {
  int32_t num_seqs;            /* B >= 0 rows */
  int32_t num_q_heads;         /* Hq, multiple of num_kv_heads; Hq/Hkv in {1,2,4,8} */
  int32_t num_kv_heads;        /* Hkv >= 1 */
  int32_t head_dim;            /* D; 128 is supported */
  int32_t block_size;          /* bs: tokens per block, one of 16, 32, 64, 128 */
  int32_t num_blocks;          /* physical blocks in each pool */
  int32_t max_blocks_per_seq;  /* row stride of block_table */
  int32_t max_seq_len;         /* host-known upper bound on seq_lens (grid planning) */
  int32_t num_workers;         /* decode work split: the flattened (row, kv head, tile)
                                  work is cut into this many equal ranges, one per
                                  wave (1 .. 65536); 0 = the library chooses */
  int32_t q_dtype;             /* pa_dtype */
  int32_t kv_dtype;            /* pa_dtype */
  int32_t out_dtype;           /* pa_dtype */
  const void *q;               /* [B][Hq][D] */
  const void *k_pool;          /* [num_blocks][Hkv][bs][D] */
  const void *v_pool;          /* [num_blocks][Hkv][bs][D] */
  const float *k_scale;        /* [Hkv], required iff kv_dtype == PA_FP8_E4M3, else NULL */
  const float *v_scale;        /* [Hkv], same rule */
  const int32_t *block_table;  /* [B][max_blocks_per_seq] */
  const int32_t *seq_lens;     /* [B], tokens in cache including the new one, >= 1 */
  float scale;                 /* softmax scale (1/sqrt(D) for standard attention); launching
                                  calls require it finite and > 0 (PA_ERR_UNSUPPORTED otherwise) */
  void *out;                   /* [B][Hq][D], out_dtype */
  void *workspace;             /* split records and partials (pa_decode_plan); NULL only when B == 0 */
  size_t workspace_bytes;
} pa_decode_args;

/* Arguments of a mixed in-flight batch, rows in three classes, in this order:
 *   [0, D)        decode rows (q_len 1), D = num_decode_rows;
 *   [D, D + V)    verify rows (1 <= q_len <= max_verify_q_len), V = num_verify_rows:
 *                 a few new tokens per row, e.g. the drafted tokens of
 *                 speculative decoding;
 *   [D + V, B)    chunked-prefill rows (q_len <= max_q_len).
 * Every row's q_len new tokens are already appended to the cache.  The class
 * only chooses the kernel; the result is the same attention for all rows. */
typedef struct pa_mixed_args {
  pa_decode_args base;         /* base.q and base.out are [total_q][Hq][D];
                                  base.seq_lens counts the row's new tokens too;
                                  base.num_workers (if nonzero) also sets the
                                  verify rows' work split */
  const int32_t *q_start_loc;  /* [num_seqs + 1] */
  int32_t total_q;             /* q_start_loc[num_seqs] */
  int32_t num_decode_rows;     /* rows with q_len == 1 placed first */
  int32_t max_q_len;           /* host-known upper bound on prefill-row q_len */
  int32_t num_verify_rows;     /* rows following the decode rows (0 = none) */
  int32_t max_verify_q_len;    /* host-known upper bound on verify-row q_len; with
                                  G = Hq/Hkv, max_verify_q_len * G <= 32 */
} pa_mixed_args;

/* Arguments of a KV append: write a step's new tokens into their cache slots
 * (each step adds one key and value per token, taking a new block when the
 * last one is full: "How does TensorRT-LLM work" (outcomeschool.com), section
 * "The paged KV cache").  The host allocator chooses the slots. */
typedef struct pa_append_args {
  int32_t num_tokens;          /* T >= 0 new tokens */
  int32_t num_kv_heads;        /* Hkv >= 1 */
  int32_t head_dim;            /* D; 128 is supported */
  int32_t block_size;          /* 16, 32, 64 or 128 */
  int32_t num_blocks;          /* physical blocks in each pool */
  int32_t src_dtype;           /* dtype of k and v: PA_F32 or PA_BF16 */
  int32_t kv_dtype;            /* pool dtype: src_dtype, or PA_FP8_E4M3 */
  const void *k;               /* [T][Hkv][D] */
  const void *v;               /* [T][Hkv][D] */
  const int32_t *slot_mapping; /* [T]: block * block_size + offset, or -1 to skip the token */
  void *k_pool;                /* [num_blocks][Hkv][bs][D], kv_dtype */
  void *v_pool;
  const float *k_scale;        /* [Hkv], required iff kv_dtype == PA_FP8_E4M3: the code stored
                                  is E4M3(x / k_scale[g]) with the quotient saturated to +-448
                                  and rounded to nearest even */
  const float *v_scale;        /* [Hkv], same rule */
} pa_append_args;

/* Arguments of a shared-prefix (cascade) decode call.  Rows that begin with the
 * same tokens can point at the same cache blocks (prefix reuse: "How does
 * TensorRT-LLM work" (outcomeschool.com), section "The paged KV cache"; block
 * reuse for a shared system prompt: "TensorRT-LLM, in depth" (aicassindra.com),
 * section "The paged KV cache and block reuse").  Consecutive decode rows are
 * grouped; the rows of a group share the first shared_len tokens of their
 * caches, held in the same physical blocks.  The call reads each shared block
 * once per group: the group's queries (up to 32 query columns per kv head) are
 * attended over the shared prefix together, each row over the rest of its own
 * cache, and the two parts are combined with the log-sum-exp identity.  The
 * result is the same attention pa_decode computes; only the bytes read differ.
 * bf16 q and KV. */
typedef struct pa_cascade_args {
  pa_decode_args base;         /* the decode rows; base.num_workers (if nonzero) sets the
                                  work split of both kernels */
  const int32_t *group_start;  /* [num_groups + 1]: group k is rows [group_start[k],
                                  group_start[k + 1]); group_start[0] = 0, strictly
                                  increasing, group_start[num_groups] = num_seqs */
  const int32_t *shared_len;   /* [num_seqs]: tokens of the row's cache its group shares:
                                  equal within a group, a multiple of block_size,
                                  0 <= shared_len < seq_len, and the first
                                  shared_len / block_size block-table entries equal
                                  across the group */
  int32_t num_groups;          /* >= 1 when num_seqs > 0 */
  int32_t max_group_rows;      /* host-known bound on rows per group; with G = Hq/Hkv,
                                  max_group_rows * G <= 32 (split larger groups) */
} pa_cascade_args;

/* Launch plan of a decode call. */
typedef struct pa_plan {
  int32_t num_workers;         /* worker waves the decode kernel runs */
  int32_t tile_tokens;         /* tokens per tile: 16 (f32, bf16 KV) or 32 (FP8 KV) */
  size_t workspace_bytes;      /* per-unit split records + partial slots */
} pa_plan;

int pa_abi_version(void);

/* Validate host-visible arguments and compute the decode plan.  The plan is a
 * pure function of (num_seqs, Hq, Hkv, kv_dtype, block_size, max_seq_len,
 * num_workers) and of the current device's compute-unit count C (read once per
 * device; 256 on MI355X): it never reads device memory and never synchronises.
 * With num_workers == 0, rows bounded by max_seq_len <= 1024 tokens (and 64
 * pages) of an fp32 or bf16 cache, at most 2C (row, kv head) units, run one
 * workgroup per unit whose waves combine their results in LDS: workspace_bytes
 * is 0 and num_workers reports those waves.  When S = min(C / units,
 * ceil(tiles / 4), 8) is at least 2 (tiles = ceil(max_seq_len / 16); at most C/2
 * units of more than 4 tiles: a unit's one workgroup would leave CUs idle), each
 * unit is instead cut over S workgroups; num_workers reports the S x units
 * pieces and the workspace takes the layout below with S x units in place of
 * the workers.  Otherwise, with num_workers == 0
 * the plan takes one worker wave per SIMD (4C), or two (8C) when no unit can
 * exceed 32 tiles or the cache is FP8, fewer for small work (at least 4 tiles
 * each, counting 4 start-up tiles per unit for fp32/bf16 caches); the
 * workspace holds, for every (row, kv head) unit,
 * the first worker covering it and their count (2 x int32), then
 * (units + workers) partial slots of Hq/Hkv x (128 + 2) fp32. */
pa_status pa_decode_plan(const pa_decode_args *a, pa_plan *plan);

/* Workspace bytes a pa_decode call with these arguments needs (the plan's
 * workspace_bytes; 0 where whole units run one workgroup each and for an empty batch).
 * The caller allocates it (the library allocates nothing) and passes it in
 * a->workspace.  Returns SIZE_MAX, with pa_last_error() set, when the host-visible
 * arguments are invalid (the same checks as pa_decode_plan).  The workspace holds
 * the split-over-the-context partials the dileepadev page names Flash-Decoding
 * ("Introduction to TensorRT-LLM", section "Core Optimization Technologies"). */
size_t pa_decode_workspace_size(const pa_decode_args *a);

/* Workspace bytes a pa_mixed call needs: its decode rows' split-K partials, its
 * verify rows' partials and, when the prefill rows make few (row, kv head, head
 * block, query tile) units -- at most half as many as the prefill workgroups
 * resident at once (2 per CU for the 4-wave workgroups, 1 for the 8-wave ones
 * that prefill rows alone may use) -- their kv pieces: up to 8 per unit, each
 * waves x 32 x (128 + 2) fp32. */
pa_status pa_mixed_workspace_size(const pa_mixed_args *a, size_t *bytes);

/* Decode attention over the paged cache: the decode kernel followed by the
 * log-sum-exp merge kernel, both queued on `stream`.  The decode kernel cuts
 * the flattened (row, kv head, tile) work into num_workers equal contiguous
 * ranges (the split over the context that the dileepadev page names
 * Flash-Decoding, section "Core Optimization Technologies").  Short rows on the
 * plan's one-workgroup-per-unit path take a single launch (see pa_decode_plan). */
pa_status pa_decode(const pa_decode_args *a, void *stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels,
 * with the split partials in a fixed 16 MiB array inside the library (one per GPU,
 * held until the process ends) instead of a caller workspace.  a->workspace and
 * a->workspace_bytes are ignored; the caller still passes q, the pools, the metadata
 * and out.  Calls needing more than 16 MiB of partials (pa_decode_workspace_size)
 * return PA_ERR_WORKSPACE_TOO_SMALL before anything is launched.  Every call on one
 * GPU uses that GPU's array, so calls that overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller.  No memory is allocated and
 * nothing is synchronised; the array's device address is looked up once per device. */
pa_status pa_decode_noalloc(const pa_decode_args *a, void *stream);

/* Debug builds of the library, compiled with PA_DEVICE_CHECKS=1 (libpa_kv_checked.so,
 * `python -m paged_kv_attention_13_amd.build --checked`), check the device-resident
 * metadata that the calls above take as a precondition, at each use: a block id read from
 * the block table outside [0, num_blocks) (the table lists which pool blocks hold a request's
 * tokens, in order: "How does TensorRT-LLM work", outcomeschool.com, section "The paged KV
 * cache"), a row length outside [1, min(max_seq_len, max_blocks_per_seq * block_size)], a
 * row's query count outside [1, its length], an append slot outside the pool.  The kernel
 * then ors a bit below into a per-GPU flags word and continues with a safe value (block 0,
 * the clamped length or count, the token skipped), so the call never reads or writes outside
 * its buffers; its results are then meaningless.  Other builds compile the checks out. */
#define PA_CHECK_BLOCK_ID 1u
#define PA_CHECK_SEQ_LEN 2u
#define PA_CHECK_Q_LEN 4u
#define PA_CHECK_SLOT 8u
/* 1 in a build with the device checks, else 0. */
int pa_device_checks(void);
/* Synchronises the current device, stores the or of the PA_CHECK_* bits recorded since the
 * last call in *flags (always 0 in other builds) and clears the word.  For tests and
 * debugging: it waits for all work on the device. */
pa_status pa_device_check_flags(uint32_t *flags);

/* The two stages of pa_decode, callable separately (e.g. to time one).  On the
 * one-workgroup-per-unit plan pa_decode_partials writes every output and
 * pa_merge_partials does nothing.  Otherwise pa_decode_partials writes `out`
 * for every (row, kv head) unit that one worker covers whole; for a unit cut by worker boundaries it writes, per
 * piece and query head, the running max m (log2 domain), the sum l of
 * exp2(s - m) and the unnormalised sum of exp2(s - m) V into the workspace,
 * plus the unit's (first worker, count) record.  pa_merge_partials combines
 * the pieces of every cut unit into `out` and leaves the other rows alone.
 * The merge must run after the partials call on the same workspace. */
pa_status pa_decode_partials(const pa_decode_args *a, void *stream);
pa_status pa_merge_partials(const pa_decode_args *a, void *stream);

/* Mixed in-flight batch: decode rows through the split-K decode kernels,
 * verify rows through the split-K MFMA multi-query kernels (bf16 q; bf16 or
 * FP8-E4M3 KV), prefill-chunk rows through the MFMA causal tile kernel (bf16 q;
 * bf16 or FP8-E4M3 KV, the codes widened exactly to bf16 as each tile is staged,
 * k_scale folded into the softmax scale and v_scale applied to the output), all
 * on `stream`; fp32 pools take decode rows only.  The workspace (pa_mixed_workspace_size) holds the decode rows'
 * split records and partials, then the verify rows', then the prefill pieces
 * (a launch of few units cuts long units' cached context into up to 8 pieces
 * and a merge kernel, also on the prefill stream, combines them). */
pa_status pa_mixed(const pa_mixed_args *a, void *stream);

/* Shared-prefix decode: the prefix kernel (one pass over each group's shared
 * blocks), the decode kernel over each row's own tokens, then the merge, all on
 * `stream`.  Workspace: pa_cascade_workspace_size.  The device-resident group
 * arrays are preconditions like the block table; pa_check_cascade_metadata
 * verifies them (and the decode preconditions) on host copies. */
pa_status pa_cascade_workspace_size(const pa_cascade_args *a, size_t *bytes);
pa_status pa_decode_cascade(const pa_cascade_args *a, void *stream);
pa_status pa_check_cascade_metadata(const pa_cascade_args *a_host);

/* Append: copy (or quantise) each token's [Hkv][D] K and V rows into
 * pool[slot / bs][:, slot % bs, :].  Precondition: -1 <= slot_mapping[t] <
 * num_blocks * block_size, no two tokens share a slot (pa_check_append_metadata
 * verifies this on a host copy).  Queued on `stream`; allocates nothing. */
pa_status pa_append(const pa_append_args *a, void *stream);
pa_status pa_check_append_metadata(const pa_append_args *a_host);

/* A decode step's append and attention together: the same results as
 * pa_append(app) followed by pa_decode(dec) on `stream`.  Token b of `app` is
 * decode row b's newest token: num_tokens == num_seqs, the two argument sets
 * describe the same pools, and slot_mapping[b] is -1 or the slot of position
 * seq_lens[b] - 1 of row b (pa_check_append_decode_metadata verifies this on
 * host copies).  When the decode plan runs workgroups per (row, kv head)
 * (rows within 1,024 tokens, at most 512 units, worker count left to the
 * library, fp32 or bf16 pools) this is one launch (plus the merge when units are
 * cut over several workgroups): a unit's first workgroup writes its row's new K/V
 * to the slot and every workgroup takes position seq_len - 1 from the new rows
 * rather than from the slot, so no part of the launch reads memory it writes.
 * Otherwise the two calls are queued one after the other.  For a decode loop whose layers each
 * append one token and attend (one launch per layer instead of two). */
pa_status pa_append_decode(const pa_append_args *app, const pa_decode_args *dec, void *stream);
pa_status pa_check_append_decode_metadata(const pa_append_args *app_host, const pa_decode_args *dec_host);

/* Synchronous CPU validation of the metadata preconditions above.  The
 * pointers block_table, seq_lens (and q_start_loc) must be HOST pointers;
 * q/pool/out pointers are not read. */
pa_status pa_check_decode_metadata(const pa_decode_args *a_host);
pa_status pa_check_mixed_metadata(const pa_mixed_args *a_host);

/* Synchronous CPU validator of a whole in-flight batch (decode rows first, then
 * verify rows, then chunked-prefill rows: "TensorRT-LLM, in depth"
 * (aicassindra.com), section "In-flight batching and the scheduler"), on HOST
 * copies of block_table, seq_lens and q_start_loc: every row's block ids in
 * [0, num_blocks) for its ceil(L / bs) blocks (the ordered per-request block
 * list of "How does TensorRT-LLM work", section "The paged KV cache"),
 * 1 <= q_len <= L <= max_seq_len, decode rows of one token at their own q
 * index, verify and prefill rows within their q_len bounds, and q_start_loc
 * running from 0 to total_q.  Returns PA_ERR_BAD_METADATA with the first
 * violation in pa_last_error().  The same check as pa_check_mixed_metadata;
 * pa_check_decode_metadata is its decode-only form. */
pa_status pa_check_metadata(const pa_mixed_args *a_host);

const char *pa_status_string(pa_status s);
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
