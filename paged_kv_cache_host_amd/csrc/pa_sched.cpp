// Iteration-level continuous batching with chunked prefill, over a pa_pool.
//
// LESSON "vLLM Serving Internals", "Continuous batching at the iteration
// level" and "What the scheduler looks like": the scheduler runs once per
// iteration; sequences that reached their end leave and free their blocks;
// waiting requests are admitted while the head of the queue fits; every
// running sequence contributes a prefill slice or one decode token.
// LESSON "Chunked prefill": prompts are consumed in slices within a
// per-iteration token budget (512 by default).
// ARTICLE "vLLM inference engine architecture" (lpnh.cn) §3.1: a running
// sequence that needs a new block takes it first and is preempted (blocks
// freed, progress reset, back of the queue) when none is free; admission is
// capped by a maximum number of running sequences, takes ceil(prompt / block)
// blocks at once, and stops at the first request that does not fit.  §3.2:
// a preempted sequence recovers by recomputation, i.e. it prefills again
// every token it knows (prompt + output so far).
//
// Order inside one step: release finished -> one decode token per
// decode-phase sequence (preempting on shortage) -> admission -> prefill
// slices in running order until the budget is spent.  The slice that
// completes a sequence's known tokens yields its next output token; the
// sequence decodes from the next step on and is finished once it produced
// its target count, being released at the start of the following step.
//
// Modes (LESSON "Use It": the four schedules its simulator compares):
//  * CHUNKED (the above): admission every iteration, prompts in slices.
//  * CONTINUOUS: admission and release every iteration, but a prompt is
//    prefilled whole in the iteration that admits it, so admission also
//    stops at the first request whose prompt does not fit what is left of
//    the iteration's token budget.  A prompt longer than the whole budget is
//    admitted into an iteration with no other prefill and sliced.
//  * STATIC: a batch is formed only when nothing runs: up to max_running
//    waiting requests in arrival order, every prompt padded to the longest
//    of the batch, all prefilled in that iteration (the padded tokens of the
//    batch may not exceed the budget, a single request excepted); members
//    that reached their target keep decoding padding tokens until the last
//    one finishes, and the batch is released together.
//  * NAIVE: STATIC with batches of one request.
//
// Prefix caching (ARTICLE §4.3; CHUNKED only): a request may carry its
// prompt's token ids.  Its admission then looks up the leading full blocks
// of the prompt, all but its last token (that token is always computed, so
// a fully cached prompt still runs the slice that yields its first output
// token), among the blocks the pool has registered by content; it needs
// fresh blocks only for the rest, and its prefill starts after the shared
// tokens.  A block is registered at the start of the step after the one
// that handed out its last prompt position as prefill: by then the caller
// has written its K/V.  Registration stops where another block already
// holds the same content, and freed blocks leave the index (pa_host.cpp).
//
// The pool is driven through its public C calls only.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

struct SSeq {
  int64_t id;
  int32_t prompt;
  int32_t target;
  int32_t pad;        // padding tokens in front of the output (static batches)
  int32_t known;      // tokens to prefill on (re)admission
  int32_t prefilled;  // of `known`, tokens handed out as prefill slices
  int32_t decoded;    // output tokens produced
  bool in_prefill;
  int32_t preemptions;
  bool has_ids;       // the prompt's token ids are known (prefix caching)
  int32_t reg_blocks; // leading blocks of the current table registered so far
};

}  // namespace

struct pa_sched {
  pa_pool* pool = nullptr;
  int32_t max_running = 0;
  int32_t budget = 0;
  int32_t block_size = 16;
  int32_t mode = PA_SCHED_CHUNKED;
  std::deque<SSeq> waiting;
  std::vector<SSeq> running;
  std::unordered_set<int64_t> known_ids;
  std::unordered_map<int64_t, std::vector<int32_t>> prompt_ids;  // requests with ids
  int64_t n_done = 0;
  int64_t preemptions = 0;
  int64_t prefix_hits = 0;  // prompt tokens found in registered blocks at admission
};

using pa::fail;

static int32_t ceil_div32(int32_t a, int32_t b) { return (a + b - 1) / b; }

extern "C" {

pa_status pa_sched_create_mode(pa_pool* pool, int32_t mode, int32_t max_running,
                               int32_t prefill_budget, int32_t block_size, pa_sched** out) {
  if (!pool || !out) return fail(PA_ERR_INVALID, "pa_sched_create: NULL argument");
  if (mode < PA_SCHED_CHUNKED || mode > PA_SCHED_NAIVE)
    return fail(PA_ERR_INVALID, "pa_sched_create: unknown mode %d", mode);
  if (max_running <= 0 || prefill_budget < 0 || block_size <= 0 ||
      (mode != PA_SCHED_CHUNKED && prefill_budget == 0))
    return fail(PA_ERR_INVALID,
                "pa_sched_create: max_running=%d prefill_budget=%d block_size=%d (mode %d)",
                max_running, prefill_budget, block_size, mode);
  pa_sched* s = new (std::nothrow) pa_sched;
  if (!s) return fail(PA_ERR_INVALID, "pa_sched_create: out of host memory");
  s->pool = pool;
  s->max_running = max_running;
  s->budget = prefill_budget;
  s->block_size = block_size;
  s->mode = mode;
  s->running.reserve(static_cast<size_t>(max_running));
  *out = s;
  return PA_OK;
}

pa_status pa_sched_create(pa_pool* pool, int32_t max_running, int32_t prefill_budget,
                          int32_t block_size, pa_sched** out) {
  return pa_sched_create_mode(pool, PA_SCHED_CHUNKED, max_running, prefill_budget, block_size,
                              out);
}

void pa_sched_destroy(pa_sched* s) { delete s; }

pa_status pa_sched_add(pa_sched* s, int64_t seq, int32_t prompt_len, int32_t target) {
  if (!s) return fail(PA_ERR_INVALID, "pa_sched_add: NULL scheduler");
  if (prompt_len < 1 || target < 1)
    return fail(PA_ERR_INVALID, "pa_sched_add: prompt_len=%d target=%d must be >= 1", prompt_len,
                target);
  if (s->known_ids.count(seq)) return fail(PA_ERR_EXISTS, "pa_sched_add: sequence %lld exists",
                                           static_cast<long long>(seq));
  s->known_ids.insert(seq);
  s->waiting.push_back(SSeq{seq, prompt_len, target, 0, prompt_len, 0, 0, true, 0, false, 0});
  return PA_OK;
}

pa_status pa_sched_add_prompt(pa_sched* s, int64_t seq, int32_t prompt_len, int32_t target,
                              const int32_t* ids) {
  if (!s) return fail(PA_ERR_INVALID, "pa_sched_add_prompt: NULL scheduler");
  if (s->mode != PA_SCHED_CHUNKED)
    return fail(PA_ERR_INVALID, "pa_sched_add_prompt: prefix caching needs the chunked mode");
  if (!ids) return fail(PA_ERR_INVALID, "pa_sched_add_prompt: NULL token ids");
  const pa_status st = pa_sched_add(s, seq, prompt_len, target);
  if (st != PA_OK) return st;
  s->waiting.back().has_ids = true;
  s->prompt_ids.emplace(seq, std::vector<int32_t>(ids, ids + prompt_len));
  return PA_OK;
}

pa_status pa_sched_step(pa_sched* s, pa_sched_batch* b) {
  if (!s || !b) return fail(PA_ERR_INVALID, "pa_sched_step: NULL argument");
  // every capacity is checked before anything changes
  const int32_t R = s->max_running;
  if (b->decode_cap < R || b->prefill_cap < R || b->event_cap < R ||
      b->prefill_slots_cap < s->budget)
    return fail(PA_ERR_INVALID,
                "pa_sched_step: capacities (decode %d, prefill %d, events %d, slots %d) below "
                "max_running=%d / budget=%d",
                b->decode_cap, b->prefill_cap, b->event_cap, b->prefill_slots_cap, R, s->budget);
  if ((R > 0 && (!b->decode_seq || !b->decode_pos || !b->decode_slot || !b->prefill_seq ||
                 !b->prefill_start || !b->prefill_len || !b->prefill_emits || !b->finished ||
                 !b->admitted || !b->preempted)) ||
      (s->budget > 0 && !b->prefill_slots))
    return fail(PA_ERR_INVALID, "pa_sched_step: NULL output array");
  b->n_decode = b->n_prefill = b->n_prefill_tokens = 0;
  b->n_finished = b->n_admitted = b->n_preempted = 0;
  pa_pool* pool = s->pool;

  // prompt blocks whose K/V the last step's slices completed join the index
  for (SSeq& q : s->running) {
    if (!q.has_ids) continue;
    const int32_t nb = std::min(q.prefilled, q.prompt) / s->block_size;
    if (nb <= q.reg_blocks) continue;
    const pa_status st =
        pa_seq_register_prefix(pool, q.id, s->prompt_ids[q.id].data(), nb * s->block_size);
    if (st != PA_OK) return st;
    q.reg_blocks = nb;
  }

  const bool batched = s->mode == PA_SCHED_STATIC || s->mode == PA_SCHED_NAIVE;
  // finished sequences leave and free their blocks; a static batch leaves
  // only as a whole
  bool batch_done = true;
  if (batched)
    for (const SSeq& q : s->running) batch_done = batch_done && !q.in_prefill && q.decoded >= q.target;
  if (batch_done) {
    size_t w = 0;
    for (size_t i = 0; i < s->running.size(); ++i) {
      SSeq& q = s->running[i];
      if (!q.in_prefill && q.decoded >= q.target) {
        if (pa_seq_release(pool, q.id) != PA_OK) return PA_ERR_UNKNOWN_SEQ;
        b->finished[b->n_finished++] = q.id;
        ++s->n_done;
        if (q.has_ids) s->prompt_ids.erase(q.id);
      } else {
        s->running[w++] = q;
      }
    }
    s->running.resize(w);
  }

  // one decode token per decode-phase sequence; preempt on shortage
  {
    size_t w = 0;
    for (size_t i = 0; i < s->running.size(); ++i) {
      SSeq q = s->running[i];
      if (q.in_prefill) {
        s->running[w++] = q;
        continue;
      }
      int32_t slot = -1;
      const pa_status st = pa_seq_append(pool, q.id, 1, &slot);
      if (st == PA_ERR_NO_BLOCKS) {
        if (pa_seq_release(pool, q.id) != PA_OK) return PA_ERR_UNKNOWN_SEQ;
        ++q.preemptions;
        ++s->preemptions;
        q.in_prefill = true;
        q.prefilled = 0;
        q.reg_blocks = 0;
        q.known = q.prompt + q.pad + q.decoded;
        s->waiting.push_back(q);
        b->preempted[b->n_preempted++] = q.id;
        continue;
      }
      if (st != PA_OK) return st;
      const int32_t k = b->n_decode++;
      b->decode_seq[k] = q.id;
      b->decode_pos[k] = q.prompt + q.pad + q.decoded - 1;
      b->decode_slot[k] = slot;
      ++q.decoded;
      s->running[w++] = q;
    }
    s->running.resize(w);
  }

  // prefill slices within the budget, in running order: first the
  // sequences that were already running, then the ones admitted below
  int32_t left = s->budget;
  auto slices = [&](size_t from) -> pa_status {
    for (size_t i = from; i < s->running.size(); ++i) {
      SSeq& q = s->running[i];
      if (!q.in_prefill || left == 0) continue;
      const int32_t n = q.known - q.prefilled < left ? q.known - q.prefilled : left;
      if (n <= 0) continue;
      const pa_status st = pa_seq_slots(pool, q.id, q.prefilled, n,
                                        b->prefill_slots + b->n_prefill_tokens);
      if (st != PA_OK) return st;
      const int32_t k = b->n_prefill++;
      b->prefill_seq[k] = q.id;
      b->prefill_start[k] = q.prefilled;
      b->prefill_len[k] = n;
      b->n_prefill_tokens += n;
      q.prefilled += n;
      left -= n;
      b->prefill_emits[k] = q.prefilled == q.known;
      if (q.prefilled == q.known) {
        q.in_prefill = false;
        ++q.decoded;
      }
    }
    return PA_OK;
  };
  const size_t n_old = s->running.size();
  pa_status st = slices(0);
  if (st != PA_OK) return st;

  // admission, head of the queue first
  if (!batched) {
    while (!s->waiting.empty() && static_cast<int32_t>(s->running.size()) < R) {
      SSeq q = s->waiting.front();
      if (q.has_ids) {
        // shared: leading full blocks of the prompt but its last token
        const int32_t* ids = s->prompt_ids[q.id].data();
        const int32_t m_len = q.prompt - 1;
        int32_t matched = 0, idle = 0;
        st = pa_pool_match_prefix(pool, ids, m_len, &matched, &idle);
        if (st != PA_OK) return st;
        // (matched blocks that are retained rather than held count as free
        // but come back into use: they are not fresh blocks)
        if (pa_pool_num_free(pool) - idle <
            ceil_div32(q.known, s->block_size) - matched / s->block_size)
          break;
        int32_t shared = 0;
        st = pa_seq_create_prefix(pool, q.id, ids, m_len, &shared);
        if (st != PA_OK) return st;
        st = pa_seq_append(pool, q.id, q.known - m_len, nullptr);
        if (st != PA_OK) return st;
        q.prefilled = shared;
        q.reg_blocks = shared / s->block_size;
        s->prefix_hits += shared;
        s->waiting.pop_front();
        s->running.push_back(q);
        b->admitted[b->n_admitted++] = q.id;
        continue;
      }
      if (pa_pool_num_free(pool) < ceil_div32(q.known, s->block_size)) break;
      // a whole prompt must fit what is left of the iteration's budget
      if (s->mode == PA_SCHED_CONTINUOUS && q.known > left && left < s->budget) break;
      st = pa_seq_create(pool, q.id, q.known);
      if (st != PA_OK) return st;
      s->waiting.pop_front();
      s->running.push_back(q);
      b->admitted[b->n_admitted++] = q.id;
      if (s->mode == PA_SCHED_CONTINUOUS) {
        st = slices(s->running.size() - 1);
        if (st != PA_OK) return st;
      }
    }
  } else if (s->running.empty()) {
    // a new batch: as many heads of the queue as fit once padded
    const int32_t cap = s->mode == PA_SCHED_NAIVE ? 1 : R;
    int32_t count = 0, padded = 0;
    while (count < cap && count < static_cast<int32_t>(s->waiting.size())) {
      const int32_t p = std::max(padded, s->waiting[count].known);
      const int64_t tokens = static_cast<int64_t>(count + 1) * p;
      const int64_t blocks = static_cast<int64_t>(count + 1) * ceil_div32(p, s->block_size);
      if (blocks > pa_pool_num_free(pool) || (count > 0 && tokens > s->budget)) break;
      padded = p;
      ++count;
    }
    for (int32_t i = 0; i < count; ++i) {
      SSeq q = s->waiting.front();
      q.pad += padded - q.known;
      q.known = padded;
      st = pa_seq_create(pool, q.id, q.known);
      if (st != PA_OK) return st;
      s->waiting.pop_front();
      s->running.push_back(q);
      b->admitted[b->n_admitted++] = q.id;
    }
  }
  if (s->mode != PA_SCHED_CONTINUOUS) {
    st = slices(n_old);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

pa_status pa_sched_stats(const pa_sched* s, pa_sched_accounting* out) {
  if (!s || !out) return fail(PA_ERR_INVALID, "pa_sched_stats: NULL argument");
  out->running = static_cast<int32_t>(s->running.size());
  out->waiting = static_cast<int32_t>(s->waiting.size());
  out->finished = s->n_done;
  out->preemptions = s->preemptions;
  out->prefix_hit_tokens = s->prefix_hits;
  out->blocks_held = 0;
  out->tokens_held = 0;
  out->unwritten = 0;
  for (const SSeq& q : s->running) {
    int32_t len = 0;
    if (pa_seq_length(s->pool, q.id, &len) != PA_OK) return PA_ERR_UNKNOWN_SEQ;
    out->blocks_held += ceil_div32(len, s->block_size);
    out->tokens_held += len;
    if (q.in_prefill) out->unwritten += q.known - q.prefilled;
  }
  return PA_OK;
}

}  // extern "C"
