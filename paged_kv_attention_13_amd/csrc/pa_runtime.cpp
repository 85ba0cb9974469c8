// Host-side paged KV cache manager and in-flight batching scheduler (C ABI in
// include/pa_runtime.h).  Plain C++, no HIP calls.
//
// Blocks: a fixed pool of equal blocks with reference counts.  A request holds
// an ordered list of blocks that grows by one block when its last block is
// full, and gives them back when it finishes ("How does TensorRT-LLM work",
// outcomeschool.com, section "The paged KV cache").  With prefix reuse, every
// block that becomes full is registered under a hash chained over all tokens
// before it; a later request whose prompt starts with the same whole blocks
// takes those blocks (reference count + 1) instead of new ones ("TensorRT-LLM,
// in depth", aicassindra.com, section "The paged KV cache and block reuse").
// Blocks whose count drops to zero go back to the free list but keep their
// registration until they are handed out for new contents, so a finished
// request's prompt can still be reused.  A match is exact: the block's tokens
// and its predecessor block are compared, not only the hash.
//
// Scheduling follows the iteration described in "TensorRT-LLM, in depth",
// section "In-flight batching and the scheduler": decoding requests first, one
// token each; then waiting requests, each taking what is left of its prompt
// (after reused blocks and earlier chunks) up to the remaining token budget.
// Readings where the description is silent: a request is never matched for its
// whole prompt (at least the prompt's last token is computed, so that it
// produces its first token); a request that has run some prefill chunks keeps
// its place at the head of the waiting queue; a decoding request skipped for
// lack of a block keeps its place among the decoding requests.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"
#include "pa_runtime.h"

namespace {

using pa::set_error;

enum State : int32_t { kWaiting = 0, kPrefilling = 1, kDecoding = 2, kFinished = 3 };

struct Block {
  int32_t ref = 0;
  bool in_free = true;        // on the free list
  bool registered = false;    // reachable through the prefix map
  uint64_t hash = 0;
  int32_t parent = -1;        // block holding the preceding tokens (-1: first block)
  std::vector<int32_t> tokens;
};

struct Request {
  int64_t id = 0;
  std::vector<int32_t> prompt;
  std::vector<int32_t> generated;
  int32_t max_new = 1;
  int32_t state = kWaiting;
  int32_t num_cached = 0;
  int32_t num_reused = 0;
  int32_t registered_blocks = 0;   // leading full blocks already registered or checked
  std::vector<int32_t> blocks;

  int32_t token_at(int32_t pos) const {
    const int32_t n = (int32_t)prompt.size();
    return pos < n ? prompt[pos] : generated[pos - n];
  }
};

struct Row {
  int64_t id;
  int32_t q_len;
};

uint64_t chain_hash(uint64_t prev, const int32_t *tok, int32_t n) {
  // 64-bit FNV-1a over the previous hash and the block's tokens
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xFF;
      h *= 1099511628211ull;
    }
  };
  mix(prev);
  for (int32_t i = 0; i < n; ++i) mix((uint64_t)(uint32_t)tok[i]);
  return h;
}

}  // namespace

struct pa_kvm {
  int32_t num_blocks = 0;
  int32_t bs = 0;
  int32_t mbps = 0;
  bool reuse = false;
  std::vector<Block> blocks;
  std::deque<int32_t> free_list;      // may hold stale entries (in_free false): skipped when popped
  int32_t free_count = 0;
  std::unordered_map<uint64_t, int32_t> prefix;   // chained hash -> block
  std::unordered_map<int64_t, Request> reqs;
  std::vector<int64_t> running;       // decoding requests, admission order
  std::deque<int64_t> waiting;        // waiting or prefilling requests, arrival order
  // the last batch
  bool pending = false;
  std::vector<Row> rows;
  std::vector<int64_t> b_ids;
  std::vector<int32_t> b_seq, b_qsl, b_table, b_slots, b_pos, b_tok;

  int32_t pop_free() {
    while (!free_list.empty()) {
      const int32_t b = free_list.front();
      free_list.pop_front();
      Block &blk = blocks[b];
      if (!blk.in_free) continue;              // taken back by a prefix match
      blk.in_free = false;
      --free_count;
      if (blk.registered) {                    // new contents: forget the old ones
        auto it = prefix.find(blk.hash);
        if (it != prefix.end() && it->second == b) prefix.erase(it);
        blk.registered = false;
      }
      blk.tokens.clear();
      blk.parent = -1;
      blk.ref = 1;
      return b;
    }
    return -1;
  }

  void release(int32_t b) {
    Block &blk = blocks[b];
    if (--blk.ref == 0) {
      blk.in_free = true;
      ++free_count;
      free_list.push_back(b);
    }
  }

  // Leading whole prompt blocks found in the prefix map (at most (prompt_len - 1) / bs).
  std::vector<int32_t> match(const Request &r) const {
    std::vector<int32_t> out;
    if (!reuse) return out;
    const int32_t nmax = ((int32_t)r.prompt.size() - 1) / bs;
    uint64_t h = 0;
    int32_t parent = -1;
    for (int32_t j = 0; j < nmax; ++j) {
      const int32_t *tok = r.prompt.data() + (size_t)j * bs;
      h = chain_hash(h, tok, bs);
      auto it = prefix.find(h);
      if (it == prefix.end()) break;
      const Block &blk = blocks[it->second];
      if (blk.parent != parent || (int32_t)blk.tokens.size() != bs ||
          !std::equal(blk.tokens.begin(), blk.tokens.end(), tok))
        break;
      out.push_back(it->second);
      parent = it->second;
    }
    return out;
  }

  // Register the request's newly full blocks (prefix reuse only).
  void register_full_blocks(Request &r) {
    const int32_t full = r.num_cached / bs;
    for (int32_t j = r.registered_blocks; j < full; ++j) {
      const int32_t b = r.blocks[j];
      Block &blk = blocks[b];
      if (!blk.registered && blk.tokens.empty()) {
        const uint64_t prev = j == 0 ? 0 : blocks[r.blocks[j - 1]].hash;
        blk.tokens.resize(bs);
        for (int32_t i = 0; i < bs; ++i) blk.tokens[i] = r.token_at(j * bs + i);
        blk.parent = j == 0 ? -1 : r.blocks[j - 1];
        blk.hash = chain_hash(prev, blk.tokens.data(), bs);
        if (reuse && prefix.find(blk.hash) == prefix.end()) {
          prefix.emplace(blk.hash, b);
          blk.registered = true;
        }
      }
    }
    r.registered_blocks = std::max(r.registered_blocks, full);
  }

  void finish(Request &r) {
    for (int32_t b : r.blocks) release(b);
    r.blocks.clear();
    r.state = kFinished;
  }
};

extern "C" {

pa_status pa_kvm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq, int32_t prefix_reuse,
                        pa_kvm **out) {
  if (!out) return set_error(PA_ERR_NULL_POINTER, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1)
    return set_error(PA_ERR_BAD_SHAPE, "num_blocks=%d, block_size=%d, max_blocks_per_seq=%d must be >= 1",
                     num_blocks, block_size, max_blocks_per_seq);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return set_error(PA_ERR_UNSUPPORTED, "num_blocks * block_size must fit in int32 slot numbers");
  pa_kvm *m = new (std::nothrow) pa_kvm;
  if (!m) return set_error(PA_ERR_BAD_SHAPE, "out of host memory");
  m->num_blocks = num_blocks;
  m->bs = block_size;
  m->mbps = max_blocks_per_seq;
  m->reuse = prefix_reuse != 0;
  m->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  m->free_count = num_blocks;
  *out = m;
  return PA_OK;
}

void pa_kvm_destroy(pa_kvm *m) { delete m; }

pa_status pa_kvm_add_request(pa_kvm *m, int64_t id, const int32_t *prompt, int32_t prompt_len,
                             int32_t max_new_tokens) {
  if (!m || (!prompt && prompt_len > 0)) return set_error(PA_ERR_NULL_POINTER, "manager or prompt is NULL");
  if (prompt_len < 1 || max_new_tokens < 1)
    return set_error(PA_ERR_BAD_SHAPE, "prompt_len=%d and max_new_tokens=%d must be >= 1", prompt_len,
                     max_new_tokens);
  const int64_t most = (int64_t)prompt_len + max_new_tokens - 1;   // the last token is never fed back
  if (most > (int64_t)m->mbps * m->bs)
    return set_error(PA_ERR_BAD_SHAPE, "request %lld needs %lld cached tokens > max_blocks_per_seq * block_size",
                     (long long)id, (long long)most);
  if (m->reqs.count(id)) return set_error(PA_ERR_BAD_SHAPE, "request id %lld already exists", (long long)id);
  Request r;
  r.id = id;
  r.prompt.assign(prompt, prompt + prompt_len);
  r.max_new = max_new_tokens;
  m->reqs.emplace(id, std::move(r));
  m->waiting.push_back(id);
  return PA_OK;
}

pa_status pa_kvm_schedule(pa_kvm *m, int32_t max_batch_size, int32_t max_num_tokens, pa_kvm_batch *batch) {
  if (!m || !batch) return set_error(PA_ERR_NULL_POINTER, "manager or batch is NULL");
  if (max_batch_size < 1 || max_num_tokens < 1)
    return set_error(PA_ERR_BAD_SHAPE, "max_batch_size=%d and max_num_tokens=%d must be >= 1", max_batch_size,
                     max_num_tokens);
  if (m->pending) return set_error(PA_ERR_BAD_SHAPE, "the previous batch was not completed");
  const int32_t bs = m->bs;
  m->rows.clear();
  int32_t budget = max_num_tokens;
  // decoding requests: one token each; one more block when the last one is full
  for (int64_t id : m->running) {
    if ((int32_t)m->rows.size() == max_batch_size || budget == 0) break;
    Request &r = m->reqs[id];
    if (r.num_cached == (int32_t)r.blocks.size() * bs) {
      const int32_t b = m->pop_free();
      if (b < 0) continue;                      // no block: skipped this iteration
      r.blocks.push_back(b);
    }
    m->rows.push_back({id, 1});
    budget -= 1;
  }
  const int32_t n_dec = (int32_t)m->rows.size();
  // waiting requests: prefill, possibly chunked
  for (int64_t id : m->waiting) {
    if ((int32_t)m->rows.size() == max_batch_size || budget == 0) break;
    Request &r = m->reqs[id];
    std::vector<int32_t> reused;
    int32_t cached = r.num_cached;
    if (r.state == kWaiting) {
      reused = m->match(r);
      cached = (int32_t)reused.size() * bs;
    }
    const int32_t chunk = std::min((int32_t)r.prompt.size() - cached, budget);
    const int32_t have = (int32_t)(r.blocks.size() + reused.size());
    const int32_t need = (cached + chunk + bs - 1) / bs - have;
    // blocks a reuse takes back from the free list count against it too
    int32_t from_free = 0;
    for (int32_t b : reused) from_free += m->blocks[b].ref == 0;
    if (need + from_free > m->free_count) break;    // cannot allocate: stop admitting
    for (int32_t b : reused) {
      Block &blk = m->blocks[b];
      if (blk.ref == 0) {
        blk.in_free = false;
        --m->free_count;
      }
      ++blk.ref;
      r.blocks.push_back(b);
    }
    if (r.state == kWaiting) {
      r.num_cached = cached;
      r.num_reused = cached;
      r.registered_blocks = (int32_t)reused.size();
      r.state = kPrefilling;
    }
    for (int32_t i = 0; i < need; ++i) r.blocks.push_back(m->pop_free());
    m->rows.push_back({id, chunk});
    budget -= chunk;
  }
  // the pass's metadata
  const int32_t B = (int32_t)m->rows.size();
  m->b_ids.assign(B, 0);
  m->b_seq.assign(B, 0);
  m->b_qsl.assign(B + 1, 0);
  m->b_table.assign((size_t)B * m->mbps, -1);
  m->b_slots.clear();
  m->b_pos.clear();
  m->b_tok.clear();
  int32_t max_q = 0, max_seq = 0;
  for (int32_t i = 0; i < B; ++i) {
    const Request &r = m->reqs[m->rows[i].id];
    const int32_t q = m->rows[i].q_len;
    m->b_ids[i] = r.id;
    m->b_seq[i] = r.num_cached + q;
    m->b_qsl[i + 1] = m->b_qsl[i] + q;
    std::copy(r.blocks.begin(), r.blocks.end(), m->b_table.begin() + (size_t)i * m->mbps);
    for (int32_t p = r.num_cached; p < r.num_cached + q; ++p) {
      m->b_slots.push_back(r.blocks[p / bs] * bs + p % bs);
      m->b_pos.push_back(p);
      m->b_tok.push_back(r.token_at(p));
    }
    if (i >= n_dec) max_q = std::max(max_q, q);
    max_seq = std::max(max_seq, m->b_seq[i]);
  }
  batch->num_rows = B;
  batch->num_decode_rows = n_dec;
  batch->total_q = m->b_qsl[B];
  batch->max_q_len = max_q;
  batch->max_seq_len = max_seq;
  batch->max_blocks_per_seq = m->mbps;
  batch->request_ids = m->b_ids.data();
  batch->seq_lens = m->b_seq.data();
  batch->q_start_loc = m->b_qsl.data();
  batch->block_table = m->b_table.data();
  batch->slot_mapping = m->b_slots.data();
  batch->positions = m->b_pos.data();
  batch->token_ids = m->b_tok.data();
  m->pending = true;
  return PA_OK;
}

pa_status pa_kvm_complete(pa_kvm *m, const int32_t *sampled) {
  if (!m) return set_error(PA_ERR_NULL_POINTER, "manager is NULL");
  if (!m->pending) return set_error(PA_ERR_BAD_SHAPE, "no scheduled batch to complete");
  if (!sampled && !m->rows.empty()) return set_error(PA_ERR_NULL_POINTER, "sampled is NULL");
  std::vector<int64_t> done;
  for (size_t i = 0; i < m->rows.size(); ++i) {
    Request &r = m->reqs[m->rows[i].id];
    r.num_cached += m->rows[i].q_len;
    m->register_full_blocks(r);
    if (r.state == kPrefilling && r.num_cached == (int32_t)r.prompt.size()) {
      r.generated.push_back(sampled[i]);
      r.state = kDecoding;
      m->waiting.erase(std::find(m->waiting.begin(), m->waiting.end(), r.id));
      m->running.push_back(r.id);
    } else if (r.state == kDecoding) {
      r.generated.push_back(sampled[i]);
    }
    if (r.state == kDecoding && (int32_t)r.generated.size() == r.max_new) done.push_back(r.id);
  }
  for (int64_t id : done) {
    m->finish(m->reqs[id]);
    m->running.erase(std::find(m->running.begin(), m->running.end(), id));
  }
  m->pending = false;
  return PA_OK;
}

int32_t pa_kvm_num_free_blocks(const pa_kvm *m) { return m ? m->free_count : 0; }

int32_t pa_kvm_num_used_blocks(const pa_kvm *m) {
  if (!m) return 0;
  int32_t n = 0;
  for (const Block &b : m->blocks) n += b.ref > 0;
  return n;
}

pa_status pa_kvm_request_info_get(const pa_kvm *m, int64_t id, pa_kvm_request_info *info) {
  if (!m || !info) return set_error(PA_ERR_NULL_POINTER, "manager or info is NULL");
  auto it = m->reqs.find(id);
  if (it == m->reqs.end()) return set_error(PA_ERR_BAD_SHAPE, "no request %lld", (long long)id);
  const Request &r = it->second;
  info->state = r.state;
  info->prompt_len = (int32_t)r.prompt.size();
  info->num_cached = r.num_cached;
  info->num_reused = r.num_reused;
  info->num_generated = (int32_t)r.generated.size();
  info->num_blocks = (int32_t)r.blocks.size();
  return PA_OK;
}

pa_status pa_kvm_generated(const pa_kvm *m, int64_t id, int32_t *tokens, int32_t cap, int32_t *n) {
  if (!m || !n) return set_error(PA_ERR_NULL_POINTER, "manager or n is NULL");
  auto it = m->reqs.find(id);
  if (it == m->reqs.end()) return set_error(PA_ERR_BAD_SHAPE, "no request %lld", (long long)id);
  const std::vector<int32_t> &g = it->second.generated;
  *n = (int32_t)g.size();
  if (tokens) std::copy(g.begin(), g.begin() + std::min<size_t>(g.size(), (size_t)std::max(cap, 0)), tokens);
  return PA_OK;
}

}  // extern "C"
