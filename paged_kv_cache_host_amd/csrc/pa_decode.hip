// pa_decode: one query token per sequence attends its paged K/V.
//
// ARTICLE "vLLM inference engine architecture" (lpnh.cn) §2.3: the kernel
// finds a query's K/V blocks through block_tables up to context_lens,
// computes scores within a block and accumulates across blocks.  Here the
// accumulation is an online softmax (running max m, running sum l,
// unnormalised output o).  The 2-block steps of a context are spread over
// the 8 waves of a work-group, whose states are merged exactly through LDS:
//     m* = max_j m_j,  l* = sum_j l_j 2^(m_j - m*),
//     out = sum_j o_j 2^(m_j - m*) / l*.
// A context longer than one work-group's chunk (2048 tokens) is cut into
// chunks; each leaves one merged partial in the workspace and a small second
// kernel applies the same merge across chunks.  (Merging inside the
// work-group keeps partial results off HBM: written in the middle of the
// read stream they cost far more than their size.)  Scores are kept in base
// 2 (s = sm_scale * log2(e) * q.k) so that the exponential is the hardware
// exp2.
//
// Grouped-query heads (query head h reads KV head h / G, G = H_q / H_kv)
// share every K/V byte: one wave computes all G heads of its KV head, so each
// K/V tile is read from HBM once per KV head.
//
// Matrix-core mapping (gfx950, wave64), one step = two 16-token blocks:
//   scores  S^T[token][head] = K[token][:] . Q^T[:][head]
//           v_mfma_f32_16x16x32_bf16, A = one block's K (16 tokens x 32 dims
//           per MFMA), B = Q^T (32 dims x 16 head columns; heads >= G are
//           zero columns).  Lane (c = l % 16, g = l / 16) receives the scores
//           of tokens 4g..4g+3 for head c.
//   output  O^T[d][head] += V^T[d][token] . P^T[token][head]
//           v_mfma_f32_16x16x16_bf16 per block: A = V^T (16 dims x 16
//           tokens), B = P^T, which is exactly the score registers (tokens
//           4g..4g+3 of head c) after the softmax update; no lane exchange.
//           The weights enter as two bf16 terms (rounded value + rounded
//           remainder), two MFMAs each, for 16 significant bits.
// Loads: a block's K tile is stored as 16-byte chunks of its 16 tokens side
// by side ([D/x][16][x]), so the K operand of one MFMA step is one 1 KiB
// contiguous read (lane = token, lane group = chunk); the V tile is stored
// token-minor ([D][16]), so a lane's 4 tokens of one dim are 8 contiguous
// bytes and a 16-dim slice of the tile is one 512-byte read.  The data is
// read once, so all K/V loads are non-temporal.
#include "pa_decode_body.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace pa {

// Persistent kernel: grid = as many work-groups as fit on the device at once.
// The work items are (sequence, KV head, chunk) for every chunk that holds
// part of a context; each work-group derives the item list from the context
// lengths in LDS, then takes items in turn from a ticket counter in the
// workspace (the next ticket is fetched when the current item's streaming
// ends, so its latency overlaps the merge).  Its waves share out the 2-block
// steps of the item's chunk and merge their running (m, l, o) through LDS.
// A context
// that fits one chunk gets its output here; longer ones leave one partial per
// chunk for the merge kernel.  The last work-group to finish resets the
// ticket counters, so they are zero again for the next call.
template <typename CacheT, int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, int32_t num_blocks, const int32_t* __restrict__ context_lens, int32_t S,
    int32_t H_q, int32_t H_kv, int32_t G, int32_t n_chunks, int32_t chunk_shift, float score_scale,
    float out_scale, int32_t* __restrict__ counters, float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  __shared__ DecodeShared<D> sh;
  decode_work<CacheT, D, BS, false>(sh, out, q, k_cache, v_cache, block_tables, max_blocks,
                                    num_blocks, context_lens, S, H_q, H_kv, G, n_chunks,
                                    chunk_shift, score_scale, out_scale, counters, ws_ml, ws_o,
                                    nullptr);
  decode_finish(counters);
}

// grid: ceil(S * H_q / 4); block: 256 (one wave per (sequence, query head)).
// Merges the chunk partials of sequences whose context spans several chunks.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, int32_t max_blocks, int32_t bs, int32_t S,
    int32_t H_q, int32_t n_chunks, int32_t chunk_shift, float out_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (idx >= static_cast<int64_t>(S) * H_q) return;
  const int seq = static_cast<int>(idx / H_q);
  const int32_t L = min(context_lens[seq], max_blocks * bs);
  const int32_t nblk = (L + kBlock - 1) / kBlock;
  const int nsp = L <= 0 ? 0 : min(n_chunks, ((nblk - 1) >> chunk_shift) + 1);
  if (nsp == 1) return;  // written by the attention kernel
  decode_merge_row<D>(out, ws_ml, ws_o, idx, nsp, n_chunks, lane, out_scale);
}

// Launches the chunk merge of a decode over S sequences (n_chunks > 1).
pa_status launch_decode_merge(hipStream_t st, void* out, const float* ws_ml, const float* ws_o,
                              const int32_t* context_lens, int32_t max_blocks, int32_t bs,
                              int32_t S, int32_t H_q, int32_t D, int32_t n_chunks, int32_t shift,
                              float out_scale) {
  const int64_t rows = static_cast<int64_t>(S) * H_q;
  auto* kern = D == 128 ? decode_merge_kernel<128> : decode_merge_kernel<64>;
  hipError_t e = launch(kDecodeMerge, kern, dim3((rows + 3) / 4), dim3(256), 0, st,
                        static_cast<uint16_t*>(out), ws_ml, ws_o, context_lens, max_blocks, bs, S,
                        H_q, n_chunks, shift, out_scale);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "decode merge launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

// Work-groups of the persistent kernel that fit on the current device at
// once (cached per device).
template <typename CacheT, int D, int BS>
static int32_t resident_work_groups() {
  static int32_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<CacheT, D, BS>, kThreads,
                                                   0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev] = cus * per_cu;
  return cached[dev];
}

template <typename CacheT, int D, int BS>
static pa_status launch_decode_mfma(hipStream_t st, void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    int32_t max_blocks, int32_t num_blocks,
                                    const int32_t* context_lens, int32_t S, int32_t H_q,
                                    int32_t H_kv, int32_t max_context_len, float sm_scale,
                                    float k_scale, float v_scale, int32_t* counters,
                                    void* partials) {
  const int32_t shift = decode_chunk_shift(S, H_kv, max_context_len);
  const int32_t n_chunks = decode_num_chunks(max_context_len, shift);
  float* ws_ml = static_cast<float*>(partials);
  float* ws_o = ws_ml + static_cast<int64_t>(S) * H_q * n_chunks * 2;
  const float score_scale = sm_scale * kLog2e * k_scale;
  const int32_t grid = resident_work_groups<CacheT, D, BS>();
  for (int32_t b = 0; b < decode_num_batches(S); ++b) {
    const int64_t s0 = static_cast<int64_t>(b) * kMaxSeqsPerLaunch;
    const int32_t sn = static_cast<int32_t>(std::min<int64_t>(kMaxSeqsPerLaunch, S - s0));
    hipError_t e = launch(kDecode, decode_kernel<CacheT, D, BS>, dim3(grid), dim3(kThreads), 0, st,
                          static_cast<uint16_t*>(out) + s0 * H_q * D,
                          static_cast<const uint16_t*>(q) + s0 * H_q * D,
                          static_cast<const typename CacheT::raw*>(k_cache),
                          static_cast<const typename CacheT::raw*>(v_cache),
                          block_tables + s0 * max_blocks, max_blocks, num_blocks, context_lens + s0,
                          sn, H_q, H_kv, H_q / H_kv, n_chunks, shift, score_scale, v_scale,
                          counters + 2 * b, ws_ml + s0 * H_q * n_chunks * 2,
                          ws_o + s0 * H_q * n_chunks * D);
    if (e != hipSuccess)
      return fail(PA_ERR_DEVICE, "pa_decode: launch failed: %s", hipGetErrorString(e));
  }
  if (n_chunks > 1)
    return launch_decode_merge(st, out, ws_ml, ws_o, context_lens, max_blocks, BS, S, H_q, D,
                               n_chunks, shift, v_scale);
  return PA_OK;
}

// Generic path (fp32 everything, or shapes outside the matrix-core path).
pa_status launch_attend_generic(hipStream_t st, void* out, pa_dtype out_dt, const void* q,
                                pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                                int32_t num_blocks, const int32_t* context_lens,
                                const int32_t* cu_q_lens, const int32_t* start_pos,
                                int32_t n_chunks, int32_t rows, int32_t H_q, int32_t H_kv,
                                int32_t D, float sm_scale, float k_scale, float v_scale);

}  // namespace pa

using namespace pa;

static bool decode_uses_mfma(pa_dtype q_dt, pa_dtype cache_dt, int32_t H_q, int32_t H_kv) {
  return q_dt == PA_BF16 && (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3) &&
         H_q / H_kv <= kMaxGroup;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                                            int32_t max_context_len) {
  if (S <= 0 || H_q <= 0 || D <= 0) return 0;
  (void)H_kv;
  // sized for the smallest chunk, so that it covers every chunk choice of
  // any call with at most these S and max_context_len
  const int64_t n_chunks = decode_num_chunks(max_context_len, kMinChunkShift);
  return decode_counter_bytes(S) + static_cast<size_t>(S) * H_q * n_chunks * (D + 2) * sizeof(float);
}

// Validation shared by pa_decode and pa_decode_noalloc; PA_OK with *run set
// when there is work to launch.
static pa_status decode_check(const char* who, void* out, pa_dtype out_dt, const void* q,
                              pa_dtype q_dt, const void* k_cache, const void* v_cache,
                              pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                              int32_t num_blocks, const int32_t* context_lens, int32_t S,
                              int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                              int32_t max_context_len, float sm_scale, float k_scale,
                              float v_scale, bool* run) {
  *run = false;
  if (bs != 8 && bs != 16 && bs != 32)
    return fail(PA_ERR_INVALID, "%s: block size %d not in {8, 16, 32}", who, bs);
  if (S < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return fail(PA_ERR_INVALID, "%s: S=%d H_q=%d H_kv=%d", who, S, H_q, H_kv);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "%s: D=%d not in {64,128}", who, D);
  if (max_blocks <= 0 || num_blocks <= 0 || max_context_len <= 0)
    return fail(PA_ERR_INVALID, "%s: max_blocks=%d num_blocks=%d max_context_len=%d", who,
                max_blocks, num_blocks, max_context_len);
  if (static_cast<int64_t>(max_blocks) * bs > INT32_MAX)
    return fail(PA_ERR_INVALID, "%s: max_blocks=%d too large", who, max_blocks);
  const bool f32 = q_dt == PA_F32 && cache_dt == PA_F32 && out_dt == PA_F32;
  const bool bf = q_dt == PA_BF16 && out_dt == PA_BF16 &&
                  (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3);
  if (!f32 && !bf)
    return fail(PA_ERR_INVALID, "%s: unsupported dtypes q=%d cache=%d out=%d", who, q_dt,
                cache_dt, out_dt);
  if (cache_dt == PA_FP8_E4M3 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
       !__builtin_isfinite(v_scale)))
    return fail(PA_ERR_INVALID, "%s: fp8 scales must be finite and > 0", who);
  if (!(sm_scale > 0.f) || !__builtin_isfinite(sm_scale))
    return fail(PA_ERR_INVALID, "%s: sm_scale must be finite and > 0", who);
  if (S == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  if (S > 65535 || H_kv > 65535)
    return fail(PA_ERR_INVALID, "%s: S=%d or H_kv=%d exceeds grid limits", who, S, H_kv);
  if (!decode_uses_mfma(q_dt, cache_dt, H_q, H_kv) && bs != kBlock)
    return fail(PA_ERR_INVALID,
                "%s: block size %d needs the matrix-core path (bf16 queries, bf16 or fp8 "
                "cache, at most 16 query heads per KV head)", who, bs);
  *run = true;
  return PA_OK;
}

// Launches a validated call; counters and partials are the workspace's two
// regions (used by the matrix-core path only).
static pa_status decode_dispatch(hipStream_t st, void* out, pa_dtype out_dt, const void* q,
                                 pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                 pa_dtype cache_dt, const int32_t* block_tables,
                                 int32_t max_blocks, int32_t num_blocks,
                                 const int32_t* context_lens, int32_t S, int32_t H_q,
                                 int32_t H_kv, int32_t D, int32_t bs, int32_t max_context_len,
                                 float sm_scale, float k_scale, float v_scale,
                                 int32_t* counters, void* partials) {
  if (decode_uses_mfma(q_dt, cache_dt, H_q, H_kv)) {
    auto by_bs = [&](auto cache_tag, auto d_tag, float ks, float vs) -> pa_status {
      using CT = decltype(cache_tag);
      constexpr int DD = decltype(d_tag)::value;
      if (bs == 8)
        return launch_decode_mfma<CT, DD, 8>(st, out, q, k_cache, v_cache, block_tables,
                                             max_blocks, num_blocks, context_lens, S, H_q, H_kv,
                                             max_context_len, sm_scale, ks, vs, counters,
                                             partials);
      if (bs == 32)
        return launch_decode_mfma<CT, DD, 32>(st, out, q, k_cache, v_cache, block_tables,
                                              max_blocks, num_blocks, context_lens, S, H_q, H_kv,
                                              max_context_len, sm_scale, ks, vs, counters,
                                              partials);
      return launch_decode_mfma<CT, DD, 16>(st, out, q, k_cache, v_cache, block_tables,
                                            max_blocks, num_blocks, context_lens, S, H_q, H_kv,
                                            max_context_len, sm_scale, ks, vs, counters,
                                            partials);
    };
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    if (cache_dt == PA_BF16)
      return D == 128 ? by_bs(BF16{}, D128{}, 1.f, 1.f) : by_bs(BF16{}, D64{}, 1.f, 1.f);
    return D == 128 ? by_bs(FP8{}, D128{}, k_scale, v_scale)
                    : by_bs(FP8{}, D64{}, k_scale, v_scale);
  }
  return launch_attend_generic(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt, block_tables,
                               max_blocks, num_blocks, context_lens, nullptr, nullptr, 0, S, H_q,
                               H_kv, D, sm_scale, k_scale, v_scale);
}

extern "C" pa_status pa_decode(void* stream, void* out, pa_dtype out_dt, const void* q,
                               pa_dtype q_dt, const void* k_cache, const void* v_cache,
                               pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                               int32_t num_blocks, const int32_t* context_lens, int32_t S,
                               int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                               int32_t max_context_len, float sm_scale, float k_scale,
                               float v_scale, void* ws, size_t ws_bytes) {
  bool run = false;
  const pa_status chk = decode_check("pa_decode", out, out_dt, q, q_dt, k_cache, v_cache,
                                     cache_dt, block_tables, max_blocks, num_blocks, context_lens,
                                     S, H_q, H_kv, D, bs, max_context_len, sm_scale, k_scale,
                                     v_scale, &run);
  if (chk != PA_OK || !run) return chk;
  int32_t* counters = nullptr;
  void* partials = nullptr;
  if (decode_uses_mfma(q_dt, cache_dt, H_q, H_kv)) {
    const size_t need = pa_decode_workspace_bytes(S, H_q, H_kv, D, max_context_len);
    if (!ws || ws_bytes < need)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace %zu bytes < %zu required", ws_bytes,
                  need);
    counters = static_cast<int32_t*>(ws);
    partials = static_cast<char*>(ws) + decode_counter_bytes(S);
  }
  return decode_dispatch(static_cast<hipStream_t>(stream), out, out_dt, q, q_dt, k_cache,
                         v_cache, cache_dt, block_tables, max_blocks, num_blocks, context_lens, S,
                         H_q, H_kv, D, bs, max_context_len, sm_scale, k_scale, v_scale, counters,
                         partials);
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: the same decode with its workspace in a file-scope device
// array, for callers that cannot allocate device memory.  The array holds a
// fixed counter region (kScratchCounterBytes, one pair of int32 per launch
// batch) followed by the split partials.  Host code never passes the array's
// name to a kernel: its device address is looked up once per device with
// hipGetSymbolAddress and kept.

namespace pa {

constexpr size_t kScratchCounterBytes = 4096;  // 512 launch batches of 4096 sequences

static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up on first use.
static pa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(PA_ERR_DEVICE, "pa_decode_noalloc: no usable current device (%s)",
                hipGetErrorString(e));
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(PA_ERR_DEVICE, "pa_decode_noalloc: scratch address lookup failed (%s)",
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// grid: 1; block: 64.  Zeroes n int32 words.
__global__ __launch_bounds__(64) void zero_words_kernel(int32_t* __restrict__ p, int32_t n) {
  for (int32_t i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

}  // namespace pa

extern "C" pa_status pa_decode_noalloc(void* stream, void* out, pa_dtype out_dt, const void* q,
                                       pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                       pa_dtype cache_dt, const int32_t* block_tables,
                                       int32_t max_blocks, int32_t num_blocks,
                                       const int32_t* context_lens, int32_t S, int32_t H_q,
                                       int32_t H_kv, int32_t D, int32_t bs,
                                       int32_t max_context_len, float sm_scale, float k_scale,
                                       float v_scale) {
  const char* who = "pa_decode_noalloc";
  bool run = false;
  const pa_status chk = decode_check(who, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt,
                                     block_tables, max_blocks, num_blocks, context_lens, S, H_q,
                                     H_kv, D, bs, max_context_len, sm_scale, k_scale, v_scale,
                                     &run);
  if (chk != PA_OK || !run) return chk;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!decode_uses_mfma(q_dt, cache_dt, H_q, H_kv))
    return decode_dispatch(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt, block_tables,
                           max_blocks, num_blocks, context_lens, S, H_q, H_kv, D, bs,
                           max_context_len, sm_scale, k_scale, v_scale, nullptr, nullptr);
  const size_t need = pa_decode_workspace_bytes(S, H_q, H_kv, D, max_context_len);
  const size_t part_need = need - decode_counter_bytes(S);
  const size_t n_counter_words = static_cast<size_t>(decode_num_batches(S)) * 2;
  if (part_need > PA_DECODE_SCRATCH_BYTES - kScratchCounterBytes ||
      n_counter_words * sizeof(int32_t) > kScratchCounterBytes)
    return fail(PA_ERR_WORKSPACE,
                "%s: the call needs %zu bytes of split partials, above the %zu this entry "
                "point holds (S=%d, H_q=%d, D=%d, max_context_len=%d); use pa_decode with a "
                "workspace", who, part_need,
                static_cast<size_t>(PA_DECODE_SCRATCH_BYTES) - kScratchCounterBytes, S, H_q, D,
                max_context_len);
  void* base = nullptr;
  const pa_status sa = scratch_address(&base);
  if (sa != PA_OK) return sa;
  int32_t* counters = static_cast<int32_t*>(base);
  // the array keeps the previous call's contents: the work counters must
  // start at zero
  zero_words_kernel<<<dim3(1), dim3(64), 0, st>>>(counters, static_cast<int32_t>(n_counter_words));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "%s: counter reset launch failed: %s", who, hipGetErrorString(e));
  return decode_dispatch(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt, block_tables,
                         max_blocks, num_blocks, context_lens, S, H_q, H_kv, D, bs,
                         max_context_len, sm_scale, k_scale, v_scale, counters,
                         static_cast<char*>(base) + kScratchCounterBytes);
}
