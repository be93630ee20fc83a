// Host batch builder of libpa (see include/pa_sched.h for what it computes
// and the passages it follows).  Host-only C++: no HIP calls.
//
// Data structures:
//   free list   intrusive doubly linked FIFO over block ids (O(1) pop, push
//               and removal of a block revived by a cache hit);
//   key maps    key -> block (hash map) and block -> key (array + flag);
//   requests    owned by id; waiting is a FIFO of ids, running a vector.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <memory>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_sched.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_bytes(uint64_t h, const uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// Key of a full block: FNV-1a over the parent key and the block's tokens,
// all little-endian.
uint64_t block_key(uint64_t parent, const int32_t* tokens, int n) {
  uint8_t buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = (uint8_t)(parent >> (8 * i));
  uint64_t h = fnv_bytes(kFnvOffset, buf, 8);
  for (int t = 0; t < n; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) buf[i] = (uint8_t)(v >> (8 * i));
    h = fnv_bytes(h, buf, 4);
  }
  return h;
}

struct Request {
  int64_t id = 0;
  std::vector<int32_t> tokens;
  int32_t prompt_len = 0, max_new = 0, generated = 0, num_computed = 0;
  std::vector<int32_t> table;
  std::vector<uint64_t> keys;  // keys of the table's full blocks
  std::vector<int32_t> host_table;  // swap-space blocks while swapped out
};

struct Entry {
  int64_t id;
  int32_t q_len, seq_len;
  std::vector<int32_t> table;
  std::vector<int64_t> slots;
};

}  // namespace

struct pa_sched {
  int32_t nb = 0, B = 0, budget = 0, chunk = 0;
  // free list
  std::vector<int32_t> next, prev;
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, free_count = 0;
  std::vector<int32_t> rc;
  std::vector<uint64_t> key_of_block;
  std::vector<uint8_t> has_key;
  std::unordered_map<uint64_t, int32_t> block_of_key;
  std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
  std::deque<int64_t> waiting;
  std::vector<Request*> running;
  int32_t finished = 0;
  std::vector<Entry> batch;
  std::vector<int64_t> preempted;
  // swap space: FIFO of free host blocks; swapped-out requests in order
  int32_t num_host = 0;
  std::deque<int32_t> host_free;
  std::deque<Request*> swapped;
  std::vector<int64_t> swapped_out;
  std::vector<std::pair<int32_t, int32_t>> swap_out, swap_in;  // (src, dst) block pairs

  void push_back(int32_t b) {
    next[b] = -1;
    prev[b] = tail;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    in_free[b] = 1;
    ++free_count;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    in_free[b] = 0;
    --free_count;
  }
  int32_t allocate() {
    const int32_t b = head;
    unlink(b);
    if (has_key[b]) {
      block_of_key.erase(key_of_block[b]);
      has_key[b] = 0;
    }
    rc[b] = 1;
    return b;
  }
  void release(Request* r) {
    for (int32_t b : r->table)
      if (--rc[b] == 0) push_back(b);
    r->table.clear();
    r->keys.clear();
  }
  int32_t blocks_needed(const Request* r, int32_t c) const {
    return (r->num_computed + c + B - 1) / B - (int32_t)r->table.size();
  }
  void register_full_blocks(Request* r) {
    while ((int32_t)r->keys.size() < r->num_computed / B) {
      const size_t i = r->keys.size();
      const uint64_t parent = r->keys.empty() ? kFnvOffset : r->keys.back();
      const uint64_t k = block_key(parent, r->tokens.data() + i * B, B);
      r->keys.push_back(k);
      const int32_t b = r->table[i];
      if (!block_of_key.count(k) && !has_key[b]) {
        block_of_key[k] = b;
        key_of_block[b] = k;
        has_key[b] = 1;
      }
    }
  }
  void schedule(Request* r, int32_t c) {
    for (int32_t n = blocks_needed(r, c); n > 0; --n) r->table.push_back(allocate());
    Entry e;
    e.id = r->id;
    e.q_len = c;
    e.slots.resize(c);
    for (int32_t j = 0; j < c; ++j) {
      const int32_t p = r->num_computed + j;
      e.slots[j] = (int64_t)r->table[p / B] * B + p % B;
    }
    r->num_computed += c;
    register_full_blocks(r);
    e.seq_len = r->num_computed;
    e.table = r->table;
    batch.push_back(std::move(e));
  }
  // Swap out when the swap space holds all the request's blocks, else
  // release them for recomputation.
  void preempt(Request* r) {
    preempted.push_back(r->id);
    if (num_host > 0 && host_free.size() >= r->table.size()) {
      for (int32_t b : r->table) {
        const int32_t h = host_free.front();
        host_free.pop_front();
        swap_out.emplace_back(b, h);
        r->host_table.push_back(h);
      }
      release(r);
      swapped.push_back(r);
      swapped_out.push_back(r->id);
      return;
    }
    release(r);
    r->num_computed = 0;
    r->prompt_len = (int32_t)r->tokens.size();
  }
  void swap_back(Request* r) {
    for (int32_t h : r->host_table) {
      const int32_t b = allocate();
      swap_in.emplace_back(h, b);
      r->table.push_back(b);
      host_free.push_back(h);
    }
    r->host_table.clear();
    register_full_blocks(r);
  }
  bool is_swapped(int64_t id) const {
    for (int64_t x : swapped_out)
      if (x == id) return true;
    return false;
  }
  // Leading full blocks with cached keys: (block, key) pairs.
  void lookup(const Request* r, std::vector<std::pair<int32_t, uint64_t>>* hits) const {
    hits->clear();
    uint64_t parent = kFnvOffset;
    const int32_t n = ((int32_t)r->tokens.size() - 1) / B;
    for (int32_t i = 0; i < n; ++i) {
      const uint64_t k = block_key(parent, r->tokens.data() + (size_t)i * B, B);
      auto it = block_of_key.find(k);
      if (it == block_of_key.end()) break;
      hits->emplace_back(it->second, k);
      parent = k;
    }
  }

  void step() {
    batch.clear();
    preempted.clear();
    swapped_out.clear();
    swap_out.clear();
    swap_in.clear();
    std::vector<Request*> decodes, prefills, still;
    for (Request* r : running) (r->num_computed >= r->prompt_len ? decodes : prefills).push_back(r);
    for (Request* r : decodes) {
      if (blocks_needed(r, 1) > free_count) {
        preempt(r);
        continue;
      }
      schedule(r, 1);
      still.push_back(r);
    }
    int64_t avail = (int64_t)budget - (int64_t)batch.size();
    if (avail < 0) avail = 0;
    for (Request* r : prefills) {
      const int64_t pending = (int64_t)r->tokens.size() - r->num_computed;
      const int32_t c = (int32_t)std::min<int64_t>(std::min<int64_t>(pending, chunk), avail);
      if (c == 0) {
        still.push_back(r);
        continue;
      }
      if (blocks_needed(r, c) > free_count) {
        preempt(r);
        continue;
      }
      schedule(r, c);
      avail -= c;
      still.push_back(r);
    }
    // requests preempted for recomputation go back to the front, in order
    for (auto it = preempted.rbegin(); it != preempted.rend(); ++it)
      if (!is_swapped(*it)) waiting.push_front(*it);
    // swapped-out requests come back, in order, when nobody was preempted
    while (!swapped.empty() && avail > 0 && preempted.empty()) {
      Request* r = swapped.front();
      const int64_t pending = (int64_t)r->tokens.size() - r->num_computed;
      const int32_t c = r->num_computed >= r->prompt_len
                            ? 1
                            : (int32_t)std::min<int64_t>(std::min<int64_t>(pending, chunk), avail);
      if ((r->num_computed + c + B - 1) / B > free_count) break;
      swapped.pop_front();
      swap_back(r);
      schedule(r, c);
      avail -= c;
      still.push_back(r);
    }
    std::vector<std::pair<int32_t, uint64_t>> hits;
    while (!waiting.empty() && avail > 0 && preempted.empty() && swapped.empty()) {
      Request* r = reqs[waiting.front()].get();
      lookup(r, &hits);
      const int32_t n_cached = (int32_t)hits.size() * B;
      const int32_t c = (int32_t)std::min<int64_t>(
          std::min<int64_t>((int64_t)r->tokens.size() - n_cached, chunk), avail);
      int32_t revive = 0;
      for (auto& h : hits) revive += rc[h.first] == 0;
      const int32_t new_blocks = (n_cached + c + B - 1) / B - (int32_t)hits.size();
      if (new_blocks > free_count - revive) break;
      waiting.pop_front();
      for (auto& h : hits) {
        if (rc[h.first] == 0) unlink(h.first);
        ++rc[h.first];
        r->table.push_back(h.first);
        r->keys.push_back(h.second);
      }
      r->num_computed = n_cached;
      schedule(r, c);
      avail -= c;
      still.push_back(r);
    }
    running.swap(still);
  }
};

extern "C" {

pa_sched* pa_sched_create(int32_t num_blocks, int32_t block_size, int32_t token_budget,
                          int32_t chunk_tokens, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0 || token_budget <= 0 || chunk_tokens <= 0)
    return nullptr;
  std::unique_ptr<pa_sched> s(new pa_sched);
  s->nb = num_blocks;
  s->B = block_size;
  s->budget = token_budget;
  s->chunk = chunk_tokens;
  s->next.assign(num_blocks, -1);
  s->prev.assign(num_blocks, -1);
  s->in_free.assign(num_blocks, 0);
  s->rc.assign(num_blocks, 0);
  s->key_of_block.assign(num_blocks, 0);
  s->has_key.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || s->in_free[b]) return nullptr;  // not a permutation
    s->push_back(b);
  }
  return s.release();
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add_request(pa_sched* s, int64_t req_id, const int32_t* prompt, int32_t prompt_len,
                         int32_t max_new_tokens) {
  if (!s || !prompt) return PA_ERR_NULL;
  if (prompt_len < 1 || max_new_tokens < 1) return PA_ERR_SHAPE;
  if (s->reqs.count(req_id)) return PA_ERR_INDEX;
  std::unique_ptr<Request> r(new Request);
  r->id = req_id;
  r->tokens.assign(prompt, prompt + prompt_len);
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  s->reqs[req_id] = std::move(r);
  s->waiting.push_back(req_id);
  return PA_OK;
}

int pa_sched_step(pa_sched* s, int32_t* num_seqs, int32_t* num_tokens, int32_t* max_blocks,
                  int32_t* num_preempted) {
  if (!s || !num_seqs || !num_tokens || !max_blocks || !num_preempted) return PA_ERR_NULL;
  s->step();
  int64_t t = 0;
  size_t mb = 0;
  for (const Entry& e : s->batch) {
    t += e.q_len;
    mb = std::max(mb, e.table.size());
  }
  *num_seqs = (int32_t)s->batch.size();
  *num_tokens = (int32_t)t;
  *max_blocks = (int32_t)mb;
  *num_preempted = (int32_t)s->preempted.size();
  return PA_OK;
}

int pa_sched_get_batch(const pa_sched* s, int64_t* req_ids, int32_t* seq_lens,
                       int32_t* query_start_loc, int32_t* block_tables,
                       int32_t max_blocks_per_seq, int32_t pad_block, int64_t* slot_mapping,
                       int64_t* preempted) {
  if (!s) return PA_ERR_NULL;
  const size_t S = s->batch.size();
  if (S > 0 && (!req_ids || !seq_lens || !query_start_loc || !block_tables || !slot_mapping))
    return PA_ERR_NULL;
  if (!s->preempted.empty() && !preempted) return PA_ERR_NULL;
  for (const Entry& e : s->batch)
    if ((int64_t)e.table.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
  if (query_start_loc) query_start_loc[0] = 0;
  int64_t t = 0;
  for (size_t i = 0; i < S; ++i) {
    const Entry& e = s->batch[i];
    req_ids[i] = e.id;
    seq_lens[i] = e.seq_len;
    int32_t* row = block_tables + i * (size_t)max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)e.table.size() ? e.table[j] : pad_block;
    memcpy(slot_mapping + t, e.slots.data(), e.slots.size() * sizeof(int64_t));
    t += e.q_len;
    query_start_loc[i + 1] = (int32_t)t;
  }
  for (size_t i = 0; i < s->preempted.size(); ++i) preempted[i] = s->preempted[i];
  return PA_OK;
}

int pa_sched_update(pa_sched* s, const int64_t* req_ids, const int32_t* tokens, int32_t n) {
  if (!s) return PA_ERR_NULL;
  if (n < 0 || (n > 0 && (!req_ids || !tokens))) return PA_ERR_SHAPE;
  std::unordered_map<int64_t, int32_t> sampled;
  for (int32_t i = 0; i < n; ++i) sampled[req_ids[i]] = tokens[i];
  // check first, so that a missing token changes nothing
  for (const Entry& e : s->batch) {
    const Request* r = s->reqs.at(e.id).get();
    if (r->num_computed == (int32_t)r->tokens.size() && r->generated < r->max_new &&
        !sampled.count(e.id))
      return PA_ERR_INDEX;
  }
  std::unordered_set<int64_t> done;
  for (const Entry& e : s->batch) {
    auto it = s->reqs.find(e.id);
    if (it == s->reqs.end()) continue;
    Request* r = it->second.get();
    if (r->num_computed < (int32_t)r->tokens.size()) continue;
    if (r->generated >= r->max_new) {
      s->release(r);
      done.insert(e.id);
      continue;
    }
    r->tokens.push_back(sampled[e.id]);
    ++r->generated;
  }
  if (!done.empty()) {
    std::vector<Request*> keep;
    for (Request* r : s->running)
      if (!done.count(r->id)) keep.push_back(r);
    s->running.swap(keep);
    for (int64_t id : done) s->reqs.erase(id);
    s->finished += (int32_t)done.size();
  }
  return PA_OK;
}

int pa_sched_block_refcounts(const pa_sched* s, int32_t* out, int32_t num_blocks) {
  if (!s || !out) return PA_ERR_NULL;
  if (num_blocks != s->nb) return PA_ERR_SHAPE;
  memcpy(out, s->rc.data(), sizeof(int32_t) * (size_t)num_blocks);
  return PA_OK;
}

int pa_sched_enable_swap(pa_sched* s, int32_t num_host_blocks) {
  if (!s) return PA_ERR_NULL;
  if (num_host_blocks < 0) return PA_ERR_SHAPE;
  if (!s->reqs.empty() || s->num_host > 0) return PA_ERR_INDEX;  // before any request, once
  s->num_host = num_host_blocks;
  for (int32_t h = 0; h < num_host_blocks; ++h) s->host_free.push_back(h);
  return PA_OK;
}

int pa_sched_get_swaps(const pa_sched* s, int32_t* num_swap_out, int32_t* num_swap_in,
                       int64_t* swap_out, int64_t* swap_in, int64_t* swapped_out_ids,
                       int32_t* num_swapped_out) {
  if (!s || !num_swap_out || !num_swap_in || !num_swapped_out) return PA_ERR_NULL;
  *num_swap_out = (int32_t)s->swap_out.size();
  *num_swap_in = (int32_t)s->swap_in.size();
  *num_swapped_out = (int32_t)s->swapped_out.size();
  if (swap_out)
    for (size_t i = 0; i < s->swap_out.size(); ++i) {
      swap_out[2 * i] = s->swap_out[i].first;
      swap_out[2 * i + 1] = s->swap_out[i].second;
    }
  if (swap_in)
    for (size_t i = 0; i < s->swap_in.size(); ++i) {
      swap_in[2 * i] = s->swap_in[i].first;
      swap_in[2 * i + 1] = s->swap_in[i].second;
    }
  if (swapped_out_ids)
    for (size_t i = 0; i < s->swapped_out.size(); ++i) swapped_out_ids[i] = s->swapped_out[i];
  return PA_OK;
}

int pa_sched_counts(const pa_sched* s, int32_t* waiting, int32_t* running, int32_t* finished) {
  if (!s || !waiting || !running || !finished) return PA_ERR_NULL;
  *waiting = (int32_t)s->waiting.size();
  *running = (int32_t)s->running.size();
  *finished = s->finished;
  return PA_OK;
}

}  // extern "C"
