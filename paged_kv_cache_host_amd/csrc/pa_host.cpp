// Host side of libpa: the FIFO block pool, per-sequence block tables, batch
// packing and error reporting.
//
// ARTICLE "vLLM inference engine architecture" (lpnh.cn) §2.2, block
// manager: every block id starts free; allocate(n) takes the first n free ids
// and fails when fewer than n are free; free(ids) appends them to the back.
// LESSON "vLLM Serving Internals", "The Concept: PagedAttention as a virtual
// memory system": a sequence's table maps logical position p to block
// table[p / bs]; one more block is added when the sequence grows past its
// blocks; blocks return to the pool when the sequence finishes.
//
// ARTICLE §4.3, prefix sharing: sequences that start with the same prefix
// reuse its blocks, read-only.  Only full blocks are shared (the sharer's
// remaining tokens, including a prefix tail that fills a partial block, get
// fresh blocks), so no sequence ever writes into a block another table
// holds.  Each block counts the tables holding it and returns to the back of
// the free list when the last of them is released.
//
// The free list is a ring buffer of int32 ids (capacity = pool size, so it
// can never overflow: a block is either in the ring or held by one or more
// tables).
//
// Prefix detection (ARTICLE §4.3: finding the requests that share a prefix
// is the scheduler's added work).  A full block whose K/V the caller has
// computed can be registered under its content: the id of the block before
// it in the sequence (none for the first) and the token ids it holds.  A
// new sequence created from its token ids walks its full blocks from the
// first and takes every block whose content is registered, stopping at the
// first that is not.  The chain through the previous block's id makes a
// match cover all earlier positions, and keys are compared in full, so no
// hash collision can produce a false match.  A block leaves the index when
// the last table holding it is released.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <iterator>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
};

// Content of a registered block: the previous block of the sequence that
// registered it (-1 for a first block) and its token ids.
struct BlockKey {
  int32_t parent = -1;
  std::vector<int32_t> tokens;
};

// FNV-1a style mix of a content, computed in place (no key object).
inline uint64_t content_hash(int32_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = 1469598103934665603ull ^ static_cast<uint32_t>(parent);
  for (int32_t i = 0; i < n; ++i) h = (h ^ static_cast<uint32_t>(tokens[i])) * 1099511628211ull;
  return h ^ (h >> 29);
}

}  // namespace

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free ids, FIFO
  int32_t head = 0;           // index of the front of the free list
  int32_t count = 0;          // number of free ids
  std::vector<int32_t> refs;  // tables holding each block (0: free)
  std::unordered_map<int64_t, Seq> seqs;
  // Registered contents: block -> its content, and content hash -> the
  // blocks registered under that hash (lookups compare the stored content,
  // so a hash collision never matches a different content).
  std::unordered_map<int32_t, BlockKey> registered;
  std::unordered_multimap<uint64_t, int32_t> index;

  int32_t at(int32_t i) const { return ring[(head + i) % num_blocks]; }
  // Prefix retention (off by default): a registered block whose last holder
  // lets go waits here, oldest first, still findable by its content, instead
  // of joining the free list; fresh blocks come from the free list first and
  // only then from the front of this list (leaving the index).
  bool retain = false;
  std::list<int32_t> lru;
  std::unordered_map<int32_t, std::list<int32_t>::iterator> lru_pos;

  int32_t available() const { return count + static_cast<int32_t>(lru.size()); }
  // Take n ids: the front of the free list, then the oldest retained blocks.
  // Caller has checked available() >= n.
  void take(int32_t n, std::vector<int32_t>& dst) {
    for (int32_t i = 0; i < n; ++i) {
      int32_t b;
      if (count > 0) {
        b = ring[head];
        head = head + 1 == num_blocks ? 0 : head + 1;
        --count;
      } else {
        b = lru.front();
        lru.pop_front();
        lru_pos.erase(b);
        unregister(b);
      }
      dst.push_back(b);
      refs[b] = 1;
    }
  }
  // A retained block found by a lookup goes back into use.
  void revive(int32_t b) {
    auto it = lru_pos.find(b);
    lru.erase(it->second);
    lru_pos.erase(it);
  }
  // Drop one reference to each id, in order; ids nobody holds any more go to
  // the back of the free list, in that order.  With retention on, the
  // registered ones are retained instead, deepest first (reverse table
  // order), so that a chain is evicted from its tail and its head, through
  // which every lookup enters it, stays findable longest.
  void give_back(const std::vector<int32_t>& ids) {
    auto at = lru.end();  // each retained block goes in front of the last one
    for (int32_t b : ids) {
      if (--refs[b] > 0) continue;
      if (retain && registered.count(b)) {
        at = lru.insert(at, b);
        lru_pos[b] = at;
        continue;
      }
      unregister(b);
      ring[(head + count) % num_blocks] = b;
      ++count;
    }
  }
  bool holds(int32_t b, int32_t parent, const int32_t* tokens) const {
    auto r = registered.find(b);
    return r != registered.end() && r->second.parent == parent &&
           std::equal(r->second.tokens.begin(), r->second.tokens.end(), tokens);
  }
  // The block registered under this content, or -1.
  int32_t find(int32_t parent, const int32_t* tokens) const {
    auto range = index.equal_range(content_hash(parent, tokens, block_size));
    for (auto it = range.first; it != range.second; ++it)
      if (holds(it->second, parent, tokens)) return it->second;
    return -1;
  }
  void add(int32_t b, int32_t parent, const int32_t* tokens) {
    registered.emplace(b, BlockKey{parent, std::vector<int32_t>(tokens, tokens + block_size)});
    index.emplace(content_hash(parent, tokens, block_size), b);
  }
  void unregister(int32_t b) {
    auto r = registered.find(b);
    if (r == registered.end()) return;
    auto range = index.equal_range(content_hash(r->second.parent, r->second.tokens.data(),
                                                block_size));
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        index.erase(it);
        break;
      }
    registered.erase(r);
  }
};

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace pa

using pa::fail;

static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

extern "C" {

int32_t pa_version(void) { return 10000; }

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                         pa_pool** out) {
  if (!out) return fail(PA_ERR_INVALID, "pa_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID, "pa_pool_create: num_blocks=%d block_size=%d", num_blocks,
                block_size);
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return fail(PA_ERR_INVALID, "pa_pool_create: out of host memory");
  try {
    p->ring.resize(static_cast<size_t>(num_blocks));
    p->refs.assign(static_cast<size_t>(num_blocks), 0);
  } catch (...) {
    delete p;
    return fail(PA_ERR_INVALID, "pa_pool_create: out of host memory for %d blocks", num_blocks);
  }
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  if (initial_free_order) {
    std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return fail(PA_ERR_INVALID,
                    "pa_pool_create: initial_free_order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
      p->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->ring[i] = i;
  }
  p->head = 0;
  p->count = num_blocks;
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_pool* pool) { return pool ? pool->available() : -1; }

int32_t pa_pool_num_seqs(const pa_pool* pool) {
  return pool ? static_cast<int32_t>(pool->seqs.size()) : -1;
}

pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n) return fail(PA_ERR_INVALID, "pa_pool_free_list: NULL argument");
  *n = pool->available();
  if (cap < pool->available() || (pool->available() > 0 && !out))
    return fail(PA_ERR_INVALID, "pa_pool_free_list: capacity %d < %d free blocks", cap,
                pool->available());
  for (int32_t i = 0; i < pool->count; ++i) out[i] = pool->at(i);
  int32_t k = pool->count;
  for (int32_t b : pool->lru) out[k++] = b;  // retained blocks, in eviction order
  return PA_OK;
}

pa_status pa_seq_create(pa_pool* pool, int64_t seq, int32_t num_tokens) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_create: pool is NULL");
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_seq_create: num_tokens=%d", num_tokens);
  if (pool->seqs.count(seq))
    return fail(PA_ERR_EXISTS, "pa_seq_create: sequence %lld exists", (long long)seq);
  int64_t need = ceil_div64(num_tokens, pool->block_size);
  if (need > pool->available())
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_create: need %lld blocks, %d free", (long long)need,
                pool->available());
  Seq s;
  s.table.reserve(static_cast<size_t>(need));
  pool->take(static_cast<int32_t>(need), s.table);
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_seq_share(pa_pool* pool, int64_t seq, int64_t src, int32_t shared_tokens,
                       int32_t num_tokens, int32_t* shared_out) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_share: pool is NULL");
  if (pool->seqs.count(seq))
    return fail(PA_ERR_EXISTS, "pa_seq_share: sequence %lld exists", (long long)seq);
  auto it = pool->seqs.find(src);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_share: unknown source sequence %lld", (long long)src);
  const Seq& from = it->second;
  if (shared_tokens < 0 || shared_tokens > from.len || num_tokens < shared_tokens)
    return fail(PA_ERR_INVALID,
                "pa_seq_share: shared_tokens=%d must lie in [0, %d] and not exceed num_tokens=%d",
                shared_tokens, from.len, num_tokens);
  const int32_t n_shared = shared_tokens / pool->block_size;
  const int64_t need = ceil_div64(num_tokens, pool->block_size) - n_shared;
  if (need > pool->available())
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_share: need %lld blocks, %d free", (long long)need,
                pool->available());
  Seq s;
  s.table.reserve(static_cast<size_t>(n_shared + need));
  for (int32_t i = 0; i < n_shared; ++i) {
    const int32_t b = from.table[i];
    s.table.push_back(b);
    ++pool->refs[b];
  }
  pool->take(static_cast<int32_t>(need), s.table);
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  if (shared_out) *shared_out = n_shared * pool->block_size;
  return PA_OK;
}

pa_status pa_seq_register_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens,
                                 int32_t n_tokens) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_register_prefix: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_register_prefix: unknown sequence %lld",
                (long long)seq);
  const Seq& s = it->second;
  if (n_tokens < 0 || n_tokens > s.len || (n_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID, "pa_seq_register_prefix: n_tokens=%d outside [0, %d] or NULL",
                n_tokens, s.len);
  const int32_t bs = pool->block_size;
  const int32_t n_full = n_tokens / bs;
  // validate first (all or nothing): a block that is already registered
  // must be registered under this content
  for (int32_t i = 0; i < n_full; ++i) {
    const int32_t b = s.table[i];
    if (pool->registered.count(b) &&
        !pool->holds(b, i ? s.table[i - 1] : -1, tokens + static_cast<int64_t>(i) * bs))
      return fail(PA_ERR_INVALID,
                  "pa_seq_register_prefix: block %d of sequence %lld is registered with other "
                  "token ids", i, (long long)seq);
  }
  for (int32_t i = 0; i < n_full; ++i) {
    const int32_t b = s.table[i];
    const int32_t parent = i ? s.table[i - 1] : -1;
    const int32_t* t = tokens + static_cast<int64_t>(i) * bs;
    const int32_t f = pool->find(parent, t);
    if (f >= 0) {
      if (f == b) continue;  // this very block
      break;  // the same content lives in another block: lookups go there
    }
    pool->add(b, parent, t);
  }
  return PA_OK;
}

pa_status pa_seq_create_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens,
                               int32_t num_tokens, int32_t* shared_out) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_create_prefix: pool is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID, "pa_seq_create_prefix: num_tokens=%d or NULL tokens", num_tokens);
  if (pool->seqs.count(seq))
    return fail(PA_ERR_EXISTS, "pa_seq_create_prefix: sequence %lld exists", (long long)seq);
  const int32_t bs = pool->block_size;
  std::vector<int32_t> matched;
  int32_t parent = -1;
  for (int32_t i = 0; i < num_tokens / bs; ++i) {
    const int32_t f = pool->find(parent, tokens + static_cast<int64_t>(i) * bs);
    if (f < 0) break;
    matched.push_back(f);
    parent = f;
  }
  // matched blocks that nobody holds (retained) come back into use and are
  // not available as fresh blocks
  int32_t idle = 0;
  for (int32_t b : matched) idle += pool->refs[b] == 0;
  const int64_t need = ceil_div64(num_tokens, bs) - static_cast<int64_t>(matched.size());
  if (need > pool->available() - idle)
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_create_prefix: need %lld blocks, %d free",
                (long long)need, pool->available() - idle);
  Seq s;
  s.table.reserve(matched.size() + static_cast<size_t>(need));
  for (int32_t b : matched) {
    s.table.push_back(b);
    if (pool->refs[b]++ == 0) pool->revive(b);
  }
  pool->take(static_cast<int32_t>(need), s.table);
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  if (shared_out) *shared_out = static_cast<int32_t>(matched.size()) * bs;
  return PA_OK;
}

pa_status pa_pool_match_prefix(const pa_pool* pool, const int32_t* tokens, int32_t num_tokens,
                               int32_t* matched_out, int32_t* retained_out) {
  if (!pool || !matched_out) return fail(PA_ERR_INVALID, "pa_pool_match_prefix: NULL argument");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID, "pa_pool_match_prefix: num_tokens=%d or NULL tokens", num_tokens);
  const int32_t bs = pool->block_size;
  int32_t parent = -1, n = 0, idle = 0;
  for (int32_t i = 0; i < num_tokens / bs; ++i) {
    const int32_t f = pool->find(parent, tokens + static_cast<int64_t>(i) * bs);
    if (f < 0) break;
    idle += pool->refs[f] == 0;
    parent = f;
    ++n;
  }
  *matched_out = n * bs;
  if (retained_out) *retained_out = idle;
  return PA_OK;
}

pa_status pa_pool_set_prefix_retention(pa_pool* pool, int32_t enable) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_pool_set_prefix_retention: pool is NULL");
  pool->retain = enable != 0;
  if (!pool->retain) {
    // retained blocks join the free list, oldest first, and leave the index
    for (int32_t b : pool->lru) {
      pool->unregister(b);
      pool->ring[(pool->head + pool->count) % pool->num_blocks] = b;
      ++pool->count;
    }
    pool->lru.clear();
    pool->lru_pos.clear();
  }
  return PA_OK;
}

int32_t pa_pool_num_retained(const pa_pool* pool) {
  return pool ? static_cast<int32_t>(pool->lru.size()) : -1;
}

int32_t pa_pool_num_registered(const pa_pool* pool) {
  return pool ? static_cast<int32_t>(pool->registered.size()) : -1;
}

pa_status pa_pool_block_refs(const pa_pool* pool, int32_t block, int32_t* refs) {
  if (!pool || !refs) return fail(PA_ERR_INVALID, "pa_pool_block_refs: NULL argument");
  if (block < 0 || block >= pool->num_blocks)
    return fail(PA_ERR_INVALID, "pa_pool_block_refs: block %d outside the pool", block);
  *refs = pool->refs[block];
  return PA_OK;
}

pa_status pa_seq_append(pa_pool* pool, int64_t seq, int32_t n_new, int32_t* slots_out) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_append: pool is NULL");
  if (n_new < 0) return fail(PA_ERR_INVALID, "pa_seq_append: n_new=%d", n_new);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_append: unknown sequence %lld", (long long)seq);
  Seq& s = it->second;
  int64_t new_len = static_cast<int64_t>(s.len) + n_new;
  if (new_len > INT32_MAX) return fail(PA_ERR_INVALID, "pa_seq_append: length overflow");
  int64_t need = ceil_div64(new_len, pool->block_size) - static_cast<int64_t>(s.table.size());
  if (need > pool->available())
    return fail(PA_ERR_NO_BLOCKS, "pa_seq_append: need %lld blocks, %d free", (long long)need,
                pool->available());
  if (need > 0) pool->take(static_cast<int32_t>(need), s.table);
  const int32_t bs = pool->block_size;
  if (slots_out) {
    for (int32_t i = 0; i < n_new; ++i) {
      int32_t p = s.len + i;
      slots_out[i] = s.table[p / bs] * bs + p % bs;
    }
  }
  s.len = static_cast<int32_t>(new_len);
  return PA_OK;
}

pa_status pa_batch_append(pa_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t n_new,
                          int32_t* slots_out, int32_t* n_done) {
  if (!pool || !n_done || n_seqs < 0 || n_new < 0 || (n_seqs > 0 && !seqs))
    return fail(PA_ERR_INVALID, "pa_batch_append: bad arguments");
  *n_done = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    pa_status st =
        pa_seq_append(pool, seqs[i], n_new,
                      slots_out ? slots_out + static_cast<int64_t>(i) * n_new : nullptr);
    if (st != PA_OK) return st;
    *n_done = i + 1;
  }
  return PA_OK;
}

pa_status pa_seq_slots(const pa_pool* pool, int64_t seq, int32_t start, int32_t n,
                       int32_t* slots_out) {
  if (!pool || (n > 0 && !slots_out)) return fail(PA_ERR_INVALID, "pa_seq_slots: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_slots: unknown sequence %lld", (long long)seq);
  const Seq& s = it->second;
  if (start < 0 || n < 0 || static_cast<int64_t>(start) + n > s.len)
    return fail(PA_ERR_INVALID, "pa_seq_slots: range [%d, %d) outside length %d", start,
                start + n, s.len);
  const int32_t bs = pool->block_size;
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = start + i;
    slots_out[i] = s.table[p / bs] * bs + p % bs;
  }
  return PA_OK;
}

pa_status pa_seq_release(pa_pool* pool, int64_t seq) {
  if (!pool) return fail(PA_ERR_INVALID, "pa_seq_release: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_release: unknown sequence %lld", (long long)seq);
  pool->give_back(it->second.table);
  pool->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_length(const pa_pool* pool, int64_t seq, int32_t* len) {
  if (!pool || !len) return fail(PA_ERR_INVALID, "pa_seq_length: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_length: unknown sequence %lld", (long long)seq);
  *len = it->second.len;
  return PA_OK;
}

pa_status pa_seq_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n) {
  if (!pool || !n) return fail(PA_ERR_INVALID, "pa_seq_block_table: NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_block_table: unknown sequence %lld", (long long)seq);
  const auto& t = it->second.table;
  *n = static_cast<int32_t>(t.size());
  if (cap < *n || (*n > 0 && !out))
    return fail(PA_ERR_INVALID, "pa_seq_block_table: capacity %d < %d", cap, *n);
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PA_OK;
}

pa_status pa_pack_batch(const pa_pool* pool, const int64_t* seqs, int32_t n_seqs,
                        int32_t max_blocks, int32_t* block_tables, int32_t* context_lens) {
  if (!pool || n_seqs < 0 || max_blocks < 0)
    return fail(PA_ERR_INVALID, "pa_pack_batch: bad arguments");
  if (n_seqs > 0 && (!seqs || !context_lens || (max_blocks > 0 && !block_tables)))
    return fail(PA_ERR_INVALID, "pa_pack_batch: NULL argument");
  // validate first so that a failure writes nothing
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "pa_pack_batch: unknown sequence %lld",
                  (long long)seqs[i]);
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return fail(PA_ERR_INVALID, "pa_pack_batch: sequence %lld holds %zu blocks > max_blocks %d",
                  (long long)seqs[i], it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Seq& s = pool->seqs.find(seqs[i])->second;
    int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(s.table.size());
    if (nb) std::memcpy(row, s.table.data(), static_cast<size_t>(nb) * sizeof(int32_t));
    for (int32_t j = nb; j < max_blocks; ++j) row[j] = -1;
    context_lens[i] = s.len;
  }
  return PA_OK;
}

pa_status pa_validate_tables(const int32_t* block_tables, const int32_t* context_lens,
                             int32_t n_seqs, int32_t max_blocks, int32_t block_size,
                             int32_t num_blocks) {
  if (n_seqs < 0 || max_blocks < 0 || block_size <= 0 || num_blocks < 0)
    return fail(PA_ERR_INVALID, "pa_validate_tables: bad sizes");
  if (n_seqs > 0 && (!context_lens || (max_blocks > 0 && !block_tables)))
    return fail(PA_ERR_INVALID, "pa_validate_tables: NULL argument");
  for (int32_t i = 0; i < n_seqs; ++i) {
    int64_t L = context_lens[i];
    if (L < 0 || L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_ERR_INVALID, "pa_validate_tables: row %d context %lld exceeds %d blocks", i,
                  (long long)L, max_blocks);
    int64_t nb = ceil_div64(L, block_size);
    const int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks;
    for (int64_t j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(PA_ERR_INVALID, "pa_validate_tables: row %d entry %lld = %d out of range", i,
                    (long long)j, row[j]);
  }
  return PA_OK;
}

}  // extern "C"
