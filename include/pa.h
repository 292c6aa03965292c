/*
 * pa.h -- C ABI of libpa, a paged-attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources of the operations (cited by title and section):
 *   LESSON   "vLLM Serving Internals: PagedAttention, Continuous Batching,
 *            Chunked Prefill" (AI Engineering from Scratch, Phase 17 Lesson
 *            04), sections "The Concept: PagedAttention as a virtual memory
 *            system", "Continuous batching at the iteration level",
 *            "Chunked prefill", "What the scheduler looks like".
 *   ARTICLE  "vLLM inference engine architecture: the PagedAttention
 *            mechanism and high-throughput inference" (lpnh.cn), sections
 *            2.2 (block manager), 2.3 (PagedAttention kernel interface),
 *            3.1 (continuous batching scheduler).
 *
 * General conventions
 *   - Every call returns a pa_status; PA_OK is 0, errors are negative.  On
 *     error nothing is launched and no state changes; pa_last_error() gives a
 *     thread-local description of the most recent error of the calling
 *     thread.
 *   - Host pointers are marked [host], device pointers [device].  Device
 *     buffers and streams belong to the caller; the library never allocates
 *     or frees device memory.  The only library-owned object is the host
 *     block pool (pa_pool), created and destroyed through this API.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Kernel calls are asynchronous on that stream: they return after the
 *     launch, and errors of the launch itself are reported as
 *     PA_ERR_DEVICE.
 *   - Element types: PA_F32 (IEEE binary32), PA_BF16 (bfloat16, stored as
 *     uint16), PA_FP8_E4M3 (OCP e4m3fn: bias 7, no infinities, max 448,
 *     stored as uint8; values are code * per-tensor fp32 scale).
 *   - The pool allocator is not thread-safe: one scheduler thread drives it,
 *     once per iteration (LESSON, "Continuous batching at the iteration
 *     level").
 *
 * KV cache layout (one layer; block size bs, KV heads H_kv, head dim D;
 * x = elements per 16 bytes of the cache type: 4 fp32, 8 bf16, 16 fp8):
 *     K cache  [num_blocks][H_kv][D/x][bs][x]   dims d..d+x-1 of the bs tokens
 *                                               of a block side by side
 *     V cache  [num_blocks][H_kv][D][bs]        a token's value is a column
 * Token position p of a sequence lives in physical block table[p / bs] at
 * offset p % bs (LESSON, "PagedAttention as a virtual memory system"); its
 * flat slot is table[p / bs] * bs + p % bs.  The ARTICLE (2.2) shapes both
 * pools [num_blocks, block_size, num_heads, head_dim]; the axis order inside
 * a pool is this library's choice: each (block, head) pair is one contiguous
 * tile, one 16-byte chunk of K for the 16 tokens is 256 contiguous bytes
 * (the operand of one matrix instruction), and values are stored token-minor
 * so that the P*V contraction reads contiguous runs of tokens.
 *
 * Supported envelope of the attention kernels (else PA_ERR_INVALID):
 *   bs == 16; D in {64, 128}; H_q % H_kv == 0; (q, cache, out) element types
 *   (f32, f32, f32), (bf16, bf16, bf16) or (bf16, fp8, bf16).  pa_decode
 *   also takes bs 8 or 32 (ARTICLE 4.1: the block size trades fragmentation
 *   against per-block overhead) with bf16 queries, a bf16 or fp8 cache and at
 *   most 16 query heads per KV head; pa_prefill_chunk takes bs 8 or 32 with
 *   bf16 queries and a bf16 or fp8 cache; pa_cache_write takes bs 8 or 32.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument, shape, dtype or envelope */
  PA_ERR_NO_BLOCKS = -2,   /* not enough free blocks; state unchanged */
  PA_ERR_UNKNOWN_SEQ = -3, /* sequence id not in the pool */
  PA_ERR_EXISTS = -4,      /* sequence id already in the pool */
  PA_ERR_DEVICE = -5,      /* HIP runtime error (launch, device query) */
  PA_ERR_WORKSPACE = -6    /* workspace missing or smaller than required */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

typedef struct pa_pool pa_pool; /* opaque host object */

/* Library version as major*10000 + minor*100 + patch. */
int32_t pa_version(void);

/* Text of the last error of the calling thread ("" if none).  The pointer
 * stays valid until the thread's next failing call. */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------
 * Host block pool -- ARTICLE 2.2 (block manager) and LESSON "PagedAttention
 * as a virtual memory system".
 *
 * The free list is FIFO: allocation takes ids from its front, release
 * appends a sequence's table to its back in table order.  Every allocation
 * is all-or-nothing: PA_ERR_NO_BLOCKS leaves the pool bit-for-bit unchanged.
 * ---------------------------------------------------------------------- */

/* Create a pool of num_blocks blocks of block_size tokens.
 * initial_free_order [host, num_blocks, may be NULL]: the initial free-list
 * order, a permutation of 0..num_blocks-1 (NULL = 0,1,..,num_blocks-1, as in
 * the ARTICLE).  The array is copied.  *out receives the pool. */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* initial_free_order, pa_pool** out);

/* Destroy a pool (NULL is accepted). */
void pa_pool_destroy(pa_pool* pool);

/* Number of free blocks (the LESSON's have_free_blocks_for test compares a
 * request's block count against this); -1 for a NULL pool. */
int32_t pa_pool_num_free(const pa_pool* pool);

/* Number of live sequences; -1 for a NULL pool. */
int32_t pa_pool_num_seqs(const pa_pool* pool);

/* Copy the free list, front first, into out [host, cap].  *n receives the
 * number of free blocks; PA_ERR_INVALID if cap is smaller. */
pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Register sequence `seq` holding num_tokens (>= 0) tokens and give it
 * ceil(num_tokens / block_size) blocks (the LESSON's
 * allocate_initial_blocks; ARTICLE 3.1 allocates a prompt's blocks at
 * admission). */
pa_status pa_seq_create(pa_pool* pool, int64_t seq, int32_t num_tokens);

/* Grow `seq` by n_new (>= 0) tokens, taking one more block each time a block
 * boundary is crossed (LESSON: "when a sequence grows past its blocks, one
 * more block is added").  slots_out [host, n_new, may be NULL] receives the
 * flat slots of the new positions. */
pa_status pa_seq_append(pa_pool* pool, int64_t seq, int32_t n_new, int32_t* slots_out);

/* Grow each of seqs[0 .. n_seqs) by n_new tokens, in order, as
 * pa_seq_append does (LESSON "Continuous batching at the iteration level":
 * every running sequence gains one token per iteration).  slots_out [host,
 * n_seqs * n_new, may be NULL]: row i receives the new slots of seqs[i].
 * Stops at the first sequence that fails; *n_done [host] receives the number
 * of sequences grown (all of them on PA_OK), and the status is that
 * sequence's error, the failing sequence itself being left unchanged. */
pa_status pa_batch_append(pa_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t n_new,
                          int32_t* slots_out, int32_t* n_done);

/* Flat slots of positions start .. start+n-1 of `seq` (all must be < the
 * sequence's length) into slots_out [host, n]. */
pa_status pa_seq_slots(const pa_pool* pool, int64_t seq, int32_t start, int32_t n,
                       int32_t* slots_out);

/* Release `seq`: it drops its hold on each of its blocks, in table order;
 * a block no other sequence holds goes to the back of the free list
 * (ARTICLE 2.2 free; LESSON release_blocks on finish). */
pa_status pa_seq_release(pa_pool* pool, int64_t seq);

/* Prefix sharing (ARTICLE 4.3: requests that start with the same
 * system-prompt prefix reuse one set of KV blocks, read-only).  Create `seq`
 * with num_tokens tokens whose first shared_tokens are the first
 * shared_tokens tokens of `src`: the shared_tokens / block_size full blocks
 * among them are src's own blocks (held by both tables from now on), the
 * rest of seq's blocks are taken fresh from the front of the free list.
 * *shared_out [host, optional] = tokens that live in shared blocks
 * ((shared_tokens / block_size) * block_size): their K/V are already in the
 * cache and must not be written again; the caller writes positions
 * shared_out .. num_tokens-1.  No sequence ever writes into a block another
 * table holds (a shared block is full; appends go to later blocks).
 * Errors (state unchanged): PA_ERR_EXISTS (seq exists), PA_ERR_UNKNOWN_SEQ
 * (src unknown), PA_ERR_INVALID (shared_tokens outside [0, length of src] or
 * above num_tokens), PA_ERR_NO_BLOCKS. */
pa_status pa_seq_share(pa_pool* pool, int64_t seq, int64_t src, int32_t shared_tokens,
                       int32_t num_tokens, int32_t* shared_out);

/* Prefix detection (ARTICLE 4.3: requests with the same system-prompt
 * prefix reuse its blocks, and finding them is the scheduler's added
 * work).  pa_seq_register_prefix declares that the K/V of positions
 * 0 .. n_tokens-1 of `seq` are in the cache and that those positions hold
 * the token ids tokens[0 .. n_tokens) [host]: each full block among them is
 * registered under its content (the id of the block before it in seq's
 * table, or none, and its block_size token ids), unless that content is
 * already registered for another block, in which case registration stops
 * there (lookups reach that other block).  A registered block leaves the
 * index when the last table holding it is released.
 * Errors (state unchanged): PA_ERR_UNKNOWN_SEQ; PA_ERR_INVALID for
 * n_tokens outside [0, length of seq], NULL tokens, or a block of seq that
 * is already registered under other token ids. */
pa_status pa_seq_register_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens,
                                 int32_t n_tokens);

/* Create `seq` for a prompt of num_tokens token ids tokens [host]: its
 * full blocks are matched from the first against the registered contents
 * (the previous block matched, or none, and the block's token ids), every
 * match is shared as by pa_seq_share, and the walk stops at the first block
 * that does not match; the remaining blocks are taken fresh from the front
 * of the free list.  *shared_out [host, optional] = tokens that live in
 * shared blocks (their K/V are in the cache; the caller writes and
 * prefills from there).  Errors (state unchanged): PA_ERR_EXISTS,
 * PA_ERR_INVALID (num_tokens < 0, NULL tokens), PA_ERR_NO_BLOCKS. */
pa_status pa_seq_create_prefix(pa_pool* pool, int64_t seq, const int32_t* tokens,
                               int32_t num_tokens, int32_t* shared_out);

/* The lookup of pa_seq_create_prefix without its effects [host]: tokens
 * (a multiple of block_size) of the leading full blocks of tokens[0 ..
 * num_tokens) whose content is registered, into *matched_out, and how many
 * of those blocks are retained rather than held (they are counted as free,
 * so a caller checking the fit subtracts them), into *retained_out
 * (optional).  Errors: PA_ERR_INVALID (NULL pool or matched_out,
 * num_tokens < 0, NULL tokens). */
pa_status pa_pool_match_prefix(const pa_pool* pool, const int32_t* tokens, int32_t num_tokens,
                               int32_t* matched_out, int32_t* retained_out);

/* Prefix retention [host; off by default, which is ARTICLE 2.2's plain FIFO
 * pool]: with enable != 0, a registered block that its last holder releases
 * is retained (still found by its content) instead of joining the free
 * list; retained blocks count as free, fresh blocks are taken from the free
 * list first and only then from the retained blocks, oldest release first,
 * each leaving the index as it is taken, and a block that
 * pa_seq_create_prefix finds while retained comes back into use.
 * pa_pool_free_list lists the free list, then the retained blocks in that
 * order.  Turning it off moves the retained blocks, oldest first, to the
 * back of the free list and out of the index.  PA_ERR_INVALID for a NULL
 * pool.  Keeping a prefix after its last request has finished is an
 * extension beyond the pages (their reuse is among running requests). */
pa_status pa_pool_set_prefix_retention(pa_pool* pool, int32_t enable);

/* Retained blocks (-1 for a NULL pool). */
int32_t pa_pool_num_retained(const pa_pool* pool);

/* Number of registered blocks (-1 for a NULL pool). */
int32_t pa_pool_num_registered(const pa_pool* pool);

/* Number of sequences holding `block` (0: free) into *refs [host]. */
pa_status pa_pool_block_refs(const pa_pool* pool, int32_t block, int32_t* refs);

/* Current token count of `seq` into *len. */
pa_status pa_seq_length(const pa_pool* pool, int64_t seq, int32_t* len);

/* Copy the block table of `seq` (ARTICLE 2.2 get_block_table) into out
 * [host, cap]; *n receives its length; PA_ERR_INVALID if cap is smaller. */
pa_status pa_seq_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n);

/* Pack a batch: block_tables [host, n_seqs * max_blocks] row i = table of
 * seqs[i] padded with -1; context_lens [host, n_seqs] = their lengths (the
 * ARTICLE 2.3 block_tables and context_lens arguments).  PA_ERR_INVALID if
 * a table is longer than max_blocks. */
pa_status pa_pack_batch(const pa_pool* pool, const int64_t* seqs, int32_t n_seqs,
                        int32_t max_blocks, int32_t* block_tables, int32_t* context_lens);

/* Host check of a packed batch: every entry of the first
 * ceil(context_lens[i] / block_size) columns of row i lies in
 * [0, num_blocks), and context_lens[i] <= max_blocks * block_size.  The
 * kernels do not trust the tables blindly (an out-of-range entry is read as
 * block 0 and an overlong context is clipped, so no access leaves the
 * buffers), but the results of such a row are meaningless; call this to
 * reject them. */
pa_status pa_validate_tables(const int32_t* block_tables, const int32_t* context_lens,
                             int32_t n_seqs, int32_t max_blocks, int32_t block_size,
                             int32_t num_blocks);

/* ------------------------------------------------------------------------
 * Cache write -- the K/V of token position p go to block table[p / bs],
 * offset p % bs (LESSON, "PagedAttention as a virtual memory system").
 *
 * k_new, v_new [device, n * H_kv * D, dtype new_dt, contiguous [n][H_kv][D]]
 * slot_mapping [device, n int32]: flat slot of each token; a slot < 0 skips
 *   the token; slots >= num_blocks * bs are also skipped (never written).
 *   Slots of one call must be distinct.
 * k_cache, v_cache [device]: the pools in the layout above, type cache_dt.
 * new_dt == cache_dt stores the bits unchanged.  new_dt == PA_BF16 with
 * cache_dt == PA_FP8_E4M3 stores code = e4m3(x * (1/scale)) with
 * 1/scale computed once in fp32 on the host, one fp32 multiply, round to
 * nearest even, magnitudes above 448 saturated to 448, NaN kept as NaN.
 * k_scale / v_scale are ignored for other caches.
 * bs: tokens per block, 8, 16 or 32 (any of the type pairs above); the
 *   staged forms below take 16.
 * ---------------------------------------------------------------------- */
pa_status pa_cache_write(void* stream, const void* k_new, const void* v_new, pa_dtype new_dt,
                         const int32_t* slot_mapping, int32_t n, void* k_cache, void* v_cache,
                         pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                         float k_scale, float v_scale);

/* ------------------------------------------------------------------------
 * Decode attention -- ARTICLE 2.3: one query token per sequence attends the
 * sequence's K/V found through block_tables up to context_lens
 * (out = softmax(sm_scale * q K^T) V, per query head; query head h reads KV
 * head h / (H_q / H_kv)).  context_lens counts the query's own token, whose
 * K/V must already be written.
 *
 * out [device, S*H_q*D, out_dt]   q [device, S*H_q*D, q_dt], both [S][H_q][D]
 * block_tables [device, S * max_blocks int32], context_lens [device, S int32],
 *   each context length in [1, max_context_len].
 * max_context_len: host-side upper bound of context_lens (sizes the split
 *   grid; no device-to-host read is needed).
 * sm_scale: softmax scale (normally 1/sqrt(D)).  k_scale, v_scale: fp8
 *   per-tensor scales (ignored otherwise).
 * bs: tokens per block, 16, or 8 / 32 on the matrix-core path (bf16 q, bf16
 *   or fp8 cache, H_q / H_kv <= 16); the cache layout above with that bs.
 * ws [device, ws_bytes]: scratch, at least pa_decode_workspace_bytes(...)
 *   bytes; else PA_ERR_WORKSPACE.  Its first bytes are work counters: the
 *   workspace must be zero-filled once before its first use, and every call
 *   leaves the counters zero again.  Calls that overlap in time must not
 *   share a workspace.
 * ---------------------------------------------------------------------- */
size_t pa_decode_workspace_bytes(int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                                 int32_t max_context_len);

pa_status pa_decode(void* stream, void* out, pa_dtype out_dt, const void* q, pa_dtype q_dt,
                    const void* k_cache, const void* v_cache, pa_dtype cache_dt,
                    const int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
                    const int32_t* context_lens, int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                    int32_t bs, int32_t max_context_len, float sm_scale, float k_scale,
                    float v_scale, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  Same arguments, operation, kernels and results as
 * pa_decode, without ws / ws_bytes: the workspace is a file-scope device
 * array of PA_DECODE_SCRATCH_BYTES (64 MiB) that each GPU the library runs
 * on holds until the process ends.  Its device address is looked up once per
 * device (with that device current) on the first call there.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * it launches a one-wave kernel that zeroes the work counters before the
 * decode kernels, since the array keeps the previous call's contents.
 *
 * Limit: the split partials of the call must fit the array less its 4 KiB
 * counter region, i.e. pa_decode_workspace_bytes(S, H_q, H_kv, D,
 * max_context_len) minus its counter bytes <= 64 MiB - 4 KiB (for example
 * 128 sequences x 64 query heads x D = 128 up to 16,384 tokens of context);
 * larger calls return PA_ERR_WORKSPACE and launch nothing.  Problems that
 * take the fp32 path use no workspace.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two threads) race and give wrong results;
 * serialise them.
 * ---------------------------------------------------------------------- */
#define PA_DECODE_SCRATCH_BYTES (64u * 1024u * 1024u)
pa_status pa_decode_noalloc(void* stream, void* out, pa_dtype out_dt, const void* q,
                            pa_dtype q_dt, const void* k_cache, const void* v_cache,
                            pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                            int32_t num_blocks, const int32_t* context_lens, int32_t S,
                            int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                            int32_t max_context_len, float sm_scale, float k_scale,
                            float v_scale);

/* ------------------------------------------------------------------------
 * Chunked-prefill attention -- LESSON "Chunked prefill": a long prompt is
 * processed as fixed-size slices (512 tokens by default), each attending
 * causally to everything before it.  Slice c holds the queries
 * q[cu_q_lens[c] .. cu_q_lens[c+1]) at absolute positions
 * start_pos[c] + i; query i sees positions 0 .. start_pos[c] + i inclusive.
 * The K/V of every one of those positions (the slice's own included) must
 * already be in the cache, reached through row c of block_tables.
 *
 * out, q [device, total_q * H_q * D], layout [total_q][H_q][D]
 * cu_q_lens [device, n_chunks + 1 int32], cu_q_lens[0] == 0, nondecreasing
 * start_pos [device, n_chunks int32], >= 0
 * block_tables [device, n_chunks * max_blocks int32]
 * max_q_len: host-side bound of the slice lengths; max_context_len: bound
 *   of start_pos[c] + q_len(c), at most bs * max_blocks.
 * bs: tokens per block, 16, or 8 / 32 with bf16 queries and a bf16 or fp8
 *   cache (the kernel's unit stays a 16-token sub-block: one block, half of
 *   a 32-token block, or two 8-token blocks).
 * ws as for pa_decode, sized by pa_prefill_workspace_bytes.
 * ---------------------------------------------------------------------- */
size_t pa_prefill_workspace_bytes(int32_t n_chunks, int32_t max_q_len, int32_t H_q,
                                  int32_t H_kv, int32_t D, int32_t max_context_len);

pa_status pa_prefill_chunk(void* stream, void* out, pa_dtype out_dt, const void* q,
                           pa_dtype q_dt, const int32_t* cu_q_lens, const int32_t* start_pos,
                           const void* k_cache, const void* v_cache, pa_dtype cache_dt,
                           const int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
                           int32_t n_chunks, int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                           int32_t max_q_len, int32_t max_context_len, float sm_scale,
                           float k_scale, float v_scale, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * Mixed-batch attention in one launch -- LESSON "What the scheduler looks
 * like": an iteration runs its decode tokens and its chunked-prefill slices
 * together as one call on the GPU.  Sequence i of the batch has the queries
 * q[cu_q_lens[i] .. cu_q_lens[i+1]) at positions seq_lens[i] - q_len(i) ..
 * seq_lens[i] - 1; query j sees positions 0 .. its own, inclusive ("Chunked
 * prefill"), through the sequence's block-table row (ARTICLE 2.3).  The K/V
 * of every such position must already be in the cache.
 *
 * The first n_decode sequences are decode rows: one query each, at rows
 * 0 .. n_decode-1 of q and out (cu_q_lens[i] == i for i <= n_decode).  The
 * next n_prefill sequences are prefill slices of 0 .. max_q_len queries.
 * The results are those of pa_decode over the decode rows (context_lens =
 * seq_lens) and pa_prefill_chunk over the slices (start_pos = seq_lens -
 * q_len), and equal them bit for bit when both take the same key-range
 * splits; one persistent kernel computes both, merging split ranges inside
 * the launch.
 *
 * out, q [device, total_q * H_q * D, bf16], layout [total_q][H_q][D]
 * cu_q_lens [device, n_decode + n_prefill + 1 int32], nondecreasing
 * seq_lens [device, n_decode + n_prefill int32]: context length of each
 *   sequence after this iteration's tokens, >= its q_len and >= 1 for a
 *   decode row
 * dec_tables [device, n_decode * dec_max_blocks int32]: row i for decode
 *   row i; pf_tables [device, n_prefill * pf_max_blocks int32]: row c for
 *   slice c (sequence n_decode + c).  One table of every sequence with
 *   stride max_blocks is passed as (tables, max_blocks) and
 *   (tables + n_decode * max_blocks, max_blocks).  Either may be NULL when
 *   its part of the batch is empty.
 * max_q_len: host-side bound of the slices' q_len; max_decode_len and
 *   max_prefill_len: bounds of seq_lens over the decode rows and the slices
 *   (sizing only; no device-to-host read), within 16 * dec_max_blocks and
 *   16 * pf_max_blocks.
 * Types: bf16 q and out with a bf16 or fp8 e4m3fn cache, D 64 or 128,
 *   bs 16, at most 16 query heads per KV head, n_decode <= 4096; other
 *   problems return PA_ERR_INVALID (pa_decode and pa_prefill_chunk take
 *   them).
 * counters [device, n_counters int32]: at least
 *   pa_attend_varlen_counters(...) work counters, zero-filled once before
 *   their first use; every call leaves them zero.  An array sized for some
 *   maxima serves every call within them.
 * ws [device, ws_bytes]: partial results of split key ranges, at least
 *   pa_attend_varlen_workspace_bytes(...) bytes (may be 0 and ws NULL when
 *   that is 0); a workspace sized for some maxima serves every call within
 *   them.  Calls that overlap in time must share neither counters nor ws.
 * ---------------------------------------------------------------------- */
int64_t pa_attend_varlen_counters(int32_t n_decode, int32_t n_prefill, int32_t H_q,
                                  int32_t H_kv, int32_t max_q_len);

size_t pa_attend_varlen_workspace_bytes(int32_t n_decode, int32_t n_prefill, int32_t H_q,
                                        int32_t H_kv, int32_t D, int32_t max_q_len,
                                        int32_t max_decode_len, int32_t max_prefill_len);

pa_status pa_attend_varlen(void* stream, void* out, pa_dtype out_dt, const void* q,
                           pa_dtype q_dt, const int32_t* cu_q_lens, const int32_t* seq_lens,
                           int32_t n_decode, int32_t n_prefill, const void* k_cache,
                           const void* v_cache, pa_dtype cache_dt, const int32_t* dec_tables,
                           int32_t dec_max_blocks, const int32_t* pf_tables,
                           int32_t pf_max_blocks, int32_t num_blocks, int32_t H_q, int32_t H_kv,
                           int32_t D, int32_t bs, int32_t max_q_len, int32_t max_decode_len,
                           int32_t max_prefill_len, float sm_scale, float k_scale,
                           float v_scale, int32_t* counters, int64_t n_counters, void* ws,
                           size_t ws_bytes);

/* ------------------------------------------------------------------------
 * Iteration-level scheduler over a pool (host).
 *
 * LESSON "Continuous batching at the iteration level", "What the scheduler
 * looks like" and "Chunked prefill"; ARTICLE 3.1 (growth before admission,
 * preemption of the sequence that cannot grow, admission capped by a
 * running-sequence limit with ceil(prompt/bs) blocks at once, stop at the
 * first request that does not fit) and 3.2 (recovery by recomputation).
 *
 * One pa_sched_step is one iteration: (1) sequences that produced their
 * target number of tokens are released; (2) every decode-phase sequence
 * appends one token (its slot is reported; on PA_ERR_NO_BLOCKS the sequence
 * is preempted: blocks freed, progress reset to prefill all of prompt +
 * output so far, queued at the back); (3) waiting sequences are admitted in
 * arrival order while fewer than max_running run and the head fits; (4)
 * prefill slices are handed out in running order until prefill_budget
 * tokens are spent.  The slice that completes a sequence's known tokens
 * yields its next output token.  The caller writes the reported tokens'
 * K/V (pa_cache_write) and runs attention before the next step.
 *
 * The scheduler drives its pool through the pa_seq_* calls; the pool must
 * not be used for other sequences meanwhile.  Not thread-safe.
 * ---------------------------------------------------------------------- */
typedef struct pa_sched pa_sched;

/* Output arrays of one step, owned by the caller (host memory).  Capacities
 * must be at least max_running (decode_cap, prefill_cap, event_cap) and
 * prefill_budget (prefill_slots_cap); pa_sched_step checks them before
 * changing anything. */
typedef struct pa_sched_batch {
  int64_t* decode_seq;     /* [decode_cap] sequences given one decode token  */
  int32_t* decode_pos;     /* [decode_cap] position of that token            */
  int32_t* decode_slot;    /* [decode_cap] its cache slot                    */
  int32_t decode_cap;
  int64_t* prefill_seq;    /* [prefill_cap] sequence of each prefill slice    */
  int32_t* prefill_start;  /* [prefill_cap] first position of the slice       */
  int32_t* prefill_len;    /* [prefill_cap] tokens in the slice               */
  int32_t* prefill_emits;  /* [prefill_cap] 1 if the slice completes the
                              sequence's known tokens (it yields an output
                              token), else 0                                  */
  int32_t prefill_cap;
  int32_t* prefill_slots;  /* [prefill_slots_cap] slots of all slices, in order */
  int32_t prefill_slots_cap;
  int64_t* finished;       /* [event_cap] released this step                 */
  int64_t* admitted;       /* [event_cap] admitted this step                  */
  int64_t* preempted;      /* [event_cap] preempted this step                 */
  int32_t event_cap;
  /* filled by pa_sched_step */
  int32_t n_decode, n_prefill, n_prefill_tokens, n_finished, n_admitted, n_preempted;
} pa_sched_batch;

/* Accounting over the running sequences (ARTICLE 2.2 / LESSON "The Concept:
 * PagedAttention as a virtual memory system"): blocks held, tokens those
 * blocks are allocated for, and of those the prompt slots not yet handed out
 * as prefill (reserved at admission, not yet written).  Internal waste =
 * 1 - tokens_held / (block_size * blocks_held). */
typedef struct pa_sched_accounting {
  int32_t running, waiting;
  int64_t finished, preemptions;
  int64_t blocks_held, tokens_held, unwritten;
  int64_t prefix_hit_tokens;  /* prompt tokens found shared at admission, in total */
} pa_sched_accounting;

/* block_size must equal the pool's.  PA_ERR_INVALID on bad sizes.  The
 * scheduler of pa_sched_create is the chunked one (PA_SCHED_CHUNKED). */
pa_status pa_sched_create(pa_pool* pool, int32_t max_running, int32_t prefill_budget,
                          int32_t block_size, pa_sched** out);

/* The four schedules the LESSON's simulator compares ("Use It"):
 *   PA_SCHED_CHUNKED     continuous batching with chunked prefill (above).
 *   PA_SCHED_CONTINUOUS  admission and release every iteration, each prompt
 *                        prefilled whole in the iteration that admits it;
 *                        admission also stops at the first request whose
 *                        known tokens exceed what is left of the iteration's
 *                        prefill_budget (a request longer than the whole
 *                        budget enters an iteration with no other prefill and
 *                        is sliced at the budget).
 *   PA_SCHED_STATIC      a batch is formed only when nothing runs: up to
 *                        max_running requests in arrival order while
 *                        count x longest prompt <= prefill_budget (one request
 *                        always) and the padded blocks fit; every prompt is
 *                        padded to the longest (padding tokens enter the cache
 *                        in front of the output: positions and slots include
 *                        them) and prefilled in that iteration; members that
 *                        reached their target keep decoding padding until the
 *                        last one does, then the batch is released together.
 *   PA_SCHED_NAIVE       PA_SCHED_STATIC with batches of one request.
 * Preemption and recomputation work as above in every mode; a preempted
 * member of a static batch keeps its padding.  prefill_budget must be >= 1
 * outside PA_SCHED_CHUNKED.  The output capacities are those of
 * pa_sched_step. */
typedef enum pa_sched_mode {
  PA_SCHED_CHUNKED = 0,
  PA_SCHED_CONTINUOUS = 1,
  PA_SCHED_STATIC = 2,
  PA_SCHED_NAIVE = 3
} pa_sched_mode;
pa_status pa_sched_create_mode(pa_pool* pool, int32_t mode, int32_t max_running,
                               int32_t prefill_budget, int32_t block_size, pa_sched** out);
void pa_sched_destroy(pa_sched* sched);
/* Queue a request (prompt_len >= 1 tokens, target >= 1 output tokens);
 * PA_ERR_EXISTS if the id was ever added. */
pa_status pa_sched_add(pa_sched* sched, int64_t seq, int32_t prompt_len, int32_t target);
/* Queue a request with its prompt's token ids (ids[prompt_len], host,
 * copied), for prefix caching (ARTICLE 4.3; PA_SCHED_CHUNKED only, else
 * PA_ERR_INVALID).  Its admission shares the leading full blocks of
 * ids[0 .. prompt_len-1) that the pool has registered by content
 * (pa_seq_create_prefix; the last prompt token is always computed), needs
 * free blocks only for the rest, and prefills from the shared count on; a
 * re-admission after preemption does the same and then grows to every
 * token it knows.  Its own full prompt blocks are registered
 * (pa_seq_register_prefix) at the start of the step after the one whose
 * slices complete them, once their K/V are in the cache. */
pa_status pa_sched_add_prompt(pa_sched* sched, int64_t seq, int32_t prompt_len, int32_t target,
                              const int32_t* ids);
pa_status pa_sched_step(pa_sched* sched, pa_sched_batch* batch);
pa_status pa_sched_stats(const pa_sched* sched, pa_sched_accounting* out);

/* ------------------------------------------------------------------------
 * pa_stage -- copy one iteration's host-built metadata (slot mappings,
 * context lengths, block tables packed by pa_batch_append / pa_pack_batch /
 * pa_sched_step) from pinned host memory to the device, as a kernel on
 * `stream`.  LESSON "Continuous batching at the iteration level": the batch
 * is rebuilt on the host every iteration; ARTICLE 2.3: the attention kernel
 * reads the block tables and context lengths from device memory.  Unlike a
 * copy-engine transfer, the kernel orders with the other kernels of the
 * stream without cross-engine waits.
 *
 * dst      [device, bytes], 4-byte aligned
 * src_host [host, bytes], 4-byte aligned, inside an allocation of pinned
 *          host memory (hipHostMalloc); else PA_ERR_INVALID.  It is read
 *          while the kernel runs: the caller must not rewrite it before the
 *          stream has passed this call (double-buffer by iteration parity).
 * bytes    multiple of 4; 0 is a no-op.
 * ---------------------------------------------------------------------- */
pa_status pa_stage(void* stream, void* dst, const void* src_host, size_t bytes);

/* pa_pinned_alias -- the host-side check every staging launch (pa_stage,
 * pa_stage_cache_write, pa_stage_decode_append) makes of its source before
 * anything is launched: src_host [host] must lie in pinned host memory
 * (hipHostMalloc); its device-side alias is written to *src_dev [host].
 * PA_ERR_INVALID (and *src_dev = NULL) for NULL or pageable memory.  Host
 * only: it never launches. */
pa_status pa_pinned_alias(const void* src_host, void** src_dev);

/* ------------------------------------------------------------------------
 * pa_stage_cache_write -- pa_stage and pa_cache_write in one launch, for an
 * iteration whose slot mapping is part of the staged metadata (LESSON
 * "Continuous batching at the iteration level": the new tokens' K/V are
 * scattered into their slots before attention reads them).  Work-groups of
 * the one kernel copy the buffer while others scatter the new tokens, the
 * latter reading the slot mapping straight from the pinned host buffer.
 *
 * dst, src_host, bytes  as for pa_stage (bytes may be 0 only when n == 0)
 * slot_offset           byte offset of the n int32 slots inside src_host;
 *                       a multiple of 4 with slot_offset + 4 n <= bytes, else
 *                       PA_ERR_INVALID.  The device copy at dst + slot_offset
 *                       holds the same slots afterwards.
 * the rest              as for pa_cache_write (types, scales, envelope and
 *                       the treatment of slots outside the pool).
 * The cache bytes and the device copy equal those of pa_stage followed by
 * pa_cache_write on the same stream.
 * ---------------------------------------------------------------------- */
pa_status pa_stage_cache_write(void* stream, void* dst, const void* src_host, size_t bytes,
                               size_t slot_offset, const void* k_new, const void* v_new,
                               pa_dtype new_dt, int32_t n, void* k_cache, void* v_cache,
                               pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv, int32_t D,
                               int32_t bs, float k_scale, float v_scale);

/* ------------------------------------------------------------------------
 * pa_stage_decode_append -- pa_stage_cache_write for a decode batch whose
 * block tables stay on the device from one iteration to the next.  ARTICLE
 * 2.2: a sequence's block table only grows, by one entry whenever its next
 * token opens a new block, and the BlockManager hands the attention kernel
 * the tables of the running sequences (2.3).  Instead of restaging whole
 * tables every iteration, the launch also enters, for each of the n new
 * tokens (one per sequence, token i belonging to row i), the block of its
 * slot at the column of its position:
 *     block_tables[i * max_blocks + (lens[i] - 1) / bs] = slots[i] / bs
 * which leaves the row unchanged unless the token opens a block.
 *
 * dst, src_host, bytes, slot_offset, k_new ... v_scale
 *               as for pa_stage_cache_write
 * lens_offset   byte offset inside src_host of the n int32 context lengths
 *               (the new token included); a multiple of 4 with
 *               lens_offset + 4 n <= bytes, else PA_ERR_INVALID.
 * block_tables  [device, n x max_blocks] int32, the batch's tables as they
 *               stood before this iteration (owned by the caller, updated in
 *               place by the kernel); NULL with n > 0 is PA_ERR_INVALID.
 * max_blocks    row stride, >= 1.
 * A token whose slot lies outside the pool, or whose length is < 1 or
 * > max_blocks * bs, leaves its row unchanged (its K/V are dropped as in
 * pa_cache_write).  Cache bytes and the staged copy equal those of
 * pa_stage_cache_write.
 * ---------------------------------------------------------------------- */
pa_status pa_stage_decode_append(void* stream, void* dst, const void* src_host, size_t bytes,
                                 size_t slot_offset, size_t lens_offset, const void* k_new,
                                 const void* v_new, pa_dtype new_dt, int32_t n, void* k_cache,
                                 void* v_cache, pa_dtype cache_dt, int32_t num_blocks,
                                 int32_t H_kv, int32_t D, int32_t bs, float k_scale,
                                 float v_scale, int32_t* block_tables, int32_t max_blocks);

/* ------------------------------------------------------------------------
 * pa_decode_append -- pa_stage_decode_append with the slots and lengths
 * already in device memory (for instance staged by pa_stage on another
 * stream while the previous iteration's attention runs), so that the launch
 * on the compute stream holds no host-memory read.  Same operation (ARTICLE
 * 2.2 / 2.3: the new tokens' K/V into their slots, a block-table entry for
 * each token that opens a block) and the same cache bytes and tables.
 *
 * slots, lens   [device, n] int32: the tokens' slots and their sequences'
 *               context lengths (new token included); owned by the caller
 * block_tables  [device, n x max_blocks] int32, updated in place
 * k_new ... v_scale as for pa_cache_write; max_blocks >= 1.
 * NULL buffers with n > 0 and the pa_cache_write argument errors are
 * PA_ERR_INVALID; n == 0 launches nothing.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_append(void* stream, const int32_t* slots, const int32_t* lens, int32_t n,
                           const void* k_new, const void* v_new, pa_dtype new_dt, void* k_cache,
                           void* v_cache, pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv,
                           int32_t D, int32_t bs, float k_scale, float v_scale,
                           int32_t* block_tables, int32_t max_blocks);

/* ------------------------------------------------------------------------
 * pa_decode_step -- one decode iteration of a batch whose block tables stay
 * on the device, in ONE launch: pa_stage_decode_append (or pa_decode_append)
 * followed by pa_decode.  LESSON "Continuous batching at the iteration
 * level": the iteration's new tokens are written into the cache before
 * attention reads it; ARTICLE 2.2: a block table grows by one entry when the
 * next token opens a block; 2.3: attention reads the tables and context
 * lengths from device memory.  The item of the persistent decode kernel that
 * streams a sequence's last block writes the new token's K/V for its KV head
 * just before reading that block, and the KV-head-0 item enters
 *     block_tables[i * max_blocks + (lens[i] - 1) / 16] = slots[i] / 16.
 * Outputs, cache bytes and tables equal those of the two launches.
 *
 * dst          [device, bytes] int32 metadata buffer holding the S slots at
 *              byte slot_offset and the S context lengths (new token
 *              included) at byte lens_offset, both multiples of 4 inside
 *              bytes, else PA_ERR_INVALID.
 * src_host     [host] pinned source of that buffer (as for pa_stage): the
 *              launch copies its first `bytes` into dst (one work-group reads
 *              the host; the others wait for it, with a bounded wait), so
 *              dst holds the staged copy afterwards.  NULL: dst already holds
 *              the metadata (for instance staged once for all the layers of
 *              an iteration) and is only read.
 * k_new, v_new [device, S x H_kv x D] bf16 (new_dt must be PA_BF16): token
 *              i's K/V, row i.
 * out, q       [device, S x H_q x D] bf16, as for pa_decode.
 * k_cache, v_cache, cache_dt (bf16 or fp8 e4m3fn with k_scale, v_scale as
 *              for pa_cache_write / pa_decode), num_blocks, H_kv, D (64 or
 *              128), bs (16 only), max_context_len (>= every length; larger
 *              lengths are attended as pa_decode attends them), sm_scale.
 * block_tables [device, S x max_blocks] int32, row i = sequence i, updated
 *              in place.
 * ws           [device, ws_bytes >= pa_decode_workspace_bytes(S, H_q, H_kv,
 *              D, max_context_len)]: the same workspace as pa_decode (its
 *              counter words zero before the first call; the launch leaves
 *              them zero).  Calls that overlap on one workspace race.
 * Limits: S <= 2048, bf16 q/out/new K/V, H_q / H_kv <= 16; else
 * PA_ERR_INVALID (use the two launches).  A token whose slot lies outside
 * the pool, or whose length is < 1 or > max_blocks * 16, is not written and
 * leaves its row unchanged (pa_stage_decode_append would still write a token
 * with a valid slot and an out-of-range length); a length < 1 also leaves the
 * output row unwritten, as pa_decode does.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_step(void* stream, int32_t* dst, const void* src_host, size_t bytes,
                         size_t slot_offset, size_t lens_offset, const void* k_new,
                         const void* v_new, pa_dtype new_dt, void* out, pa_dtype out_dt,
                         const void* q, pa_dtype q_dt, void* k_cache, void* v_cache,
                         pa_dtype cache_dt, int32_t* block_tables, int32_t max_blocks,
                         int32_t num_blocks, int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                         int32_t bs, int32_t max_context_len, float sm_scale, float k_scale,
                         float v_scale, void* ws, size_t ws_bytes);

/* pa_decode_step_set_spin_limit -- testing aid: the number of polls
 * (each followed by a short sleep) a work-group of later pa_decode_step
 * launches makes for the staged metadata before it takes no work and ends
 * (default 65536).  A tiny limit forces that path, where work-group 0 and
 * any work-group that did see the flag serve the whole queue; the results
 * are the same.  polls < 1 is PA_ERR_INVALID.  Process-wide, host only. */
pa_status pa_decode_step_set_spin_limit(int32_t polls);

/* ------------------------------------------------------------------------
 * Kernel timing (instrumentation, off by default).  Each launch of a
 * selected kernel carries a pair of HIP events attached to the launch
 * (hipExtLaunchKernel), which take that kernel's start and end times (up to
 * 4096 launches per kernel between resets).  The events cost the stream a
 * few microseconds per timed launch.  Kernel names and their bits:
 * "cache_write" 1, "decode" 2, "decode_merge" 4, "prefill" 8,
 * "prefill_merge" 16, "generic" 32, "stage" 64, "stage_cache_write" 128,
 * "varlen" 256, "decode_step" 512.
 * ---------------------------------------------------------------------- */

/* Time the kernels whose bits are set in `mask` (-1: all, 0: none): of each
 * selected kernel, the launches 0, every, 2 * every, ... counted from this
 * call (every >= 1, else PA_ERR_INVALID).  Either way the kept launches are
 * forgotten.  The events of a selected kernel's first 64 timed launches are
 * created by this call (later ones on first use), so enable timing before,
 * not inside, the region being timed.  Call it with no timed launch of the
 * previous recording still in flight (its events are reused). */
pa_status pa_timing_enable(int32_t mask, int32_t every);

/* Wait for the recorded launches of `kernel` [host string] and report their
 * number, mean and total duration in microseconds (each [host]). */
pa_status pa_timing_query(const char* kernel, int32_t* count, float* mean_us, float* total_us);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
