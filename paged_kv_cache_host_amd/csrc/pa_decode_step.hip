// pa_decode_step: one decode iteration of a batch whose block tables stay
// on the device, in one launch: the new tokens' K/V into their slots, the
// block-table entry of each token that opens a block, and decode attention
// over the grown contexts.
//
// LESSON "Continuous batching at the iteration level": each iteration's new
// tokens are written into the cache before attention reads it.  ARTICLE
// "vLLM inference engine architecture" §2.2: a sequence's block table grows
// by one entry when its next token opens a block; §2.3: the attention kernel
// reads the tables and context lengths from device memory.
//
// The attention is pa_decode's persistent kernel (pa_decode_body.h) with the
// append folded into its work items: the item that streams a sequence's
// last block (its last chunk, one per KV head) writes that KV head's new K/V
// row into the slot, from the wave that reads the block, right before that
// wave's loads of it; the KV-head-0 item enters the block into the table.
// The other KV heads' and chunks' items read nothing the append writes, so
// no work-group waits for another, and the cache bytes, tables and outputs
// equal those of pa_stage_decode_append (or pa_decode_append) followed by
// pa_decode.
//
// The batch's slots and context lengths lie in one int32 buffer, read by
// the work-groups from its device twin `dst`.  With a pinned host source,
// work-group 0 first copies the buffer into `dst` (system-scope loads: one
// host read for the launch instead of one per work-group) and publishes the
// copy through a flag in the workspace (agent-scope release); every other
// work-group polls the flag (acquire) before it starts.  The poll is
// bounded: a work-group that has not seen the flag after spin_limit polls
// takes no work and ends (work-group 0 and the others drain the work
// queue), so the launch ends whatever the order in which its work-groups
// run.
#include "pa_decode_body.h"

#include <algorithm>
#include <atomic>

namespace pa {

constexpr int32_t kStepSpins = 1 << 16;  // flag polls (each followed by a short sleep)

// The poll limit the launches use (kStepSpins unless a test lowers it).
static std::atomic<int32_t> g_step_spins{kStepSpins};
// Sequences per launch: their lengths are kept in LDS (8 KiB, which keeps
// the d = 64 kernel at two work-groups per CU).
constexpr int32_t kStepMaxSeqs = 2048;

template <int D>
struct StepShared {
  DecodeShared<D> d;
  int32_t lens[kStepMaxSeqs];  // the context lengths, read by every item
  int32_t ok;
};

// Persistent grid (as many work-groups as fit at once); block kThreads.
// counters[0..1]: pa_decode's tickets; counters[2]: the staging flag.  The
// last work-group to finish clears all three.
template <typename CacheT, int D>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    int32_t* dst, const int32_t* src, int32_t n_words, int32_t slot_word, int32_t lens_word,
    int32_t spin_limit, uint16_t* __restrict__ out, const uint16_t* __restrict__ q, typename CacheT::raw* k_cache,
    typename CacheT::raw* v_cache, int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
    int32_t S, int32_t H_q, int32_t H_kv, int32_t G, int32_t n_chunks, int32_t chunk_shift,
    float score_scale, float out_scale, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, float k_inv, float v_inv, int32_t* __restrict__ counters,
    float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  __shared__ StepShared<D> sh;
  const int tid = threadIdx.x;
  int32_t* flag = counters + 2;
  if (src != nullptr) {
    if (blockIdx.x == 0) {
      for (int32_t i = tid; i < n_words; i += kThreads)
        dst[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      // every wave's copy is published by the barrier and thread 0's
      // agent-scope release
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (tid == 0) {
        int32_t ok = 0;
        for (int32_t n = 0; n < spin_limit; ++n) {
          ok = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (ok) break;
          __builtin_amdgcn_s_sleep(1);
        }
        if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        sh.ok = ok;
      }
      __syncthreads();
      if (!sh.ok) {
        decode_finish(counters, 3);
        return;
      }
    }
  }
  for (int32_t i = tid; i < S; i += kThreads) sh.lens[i] = dst[lens_word + i];
  __syncthreads();
  DecodeAppend<CacheT> ap;
  ap.slots = dst + slot_word;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.tables = block_tables;
  ap.k_inv = k_inv;
  ap.v_inv = v_inv;
  decode_work<CacheT, D, kBlock, false, true>(sh.d, out, q, k_cache, v_cache, block_tables,
                                              max_blocks, num_blocks, sh.lens, S, H_q,
                                              H_kv, G, n_chunks, chunk_shift, score_scale,
                                              out_scale, counters, ws_ml, ws_o, nullptr, ap);
  decode_finish(counters, 3);
}

// Work-groups of the step kernel that fit on the current device at once
// (cached per device).
template <typename CacheT, int D>
static int32_t step_work_groups() {
  static int32_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<CacheT, D>,
                                                   kThreads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev] = cus * per_cu;
  return cached[dev];
}

pa_status launch_decode_merge(hipStream_t st, void* out, const float* ws_ml, const float* ws_o,
                              const int32_t* context_lens, int32_t max_blocks, int32_t bs,
                              int32_t S, int32_t H_q, int32_t D, int32_t n_chunks, int32_t shift,
                              float out_scale);

struct StepArgs {
  int32_t* dst;
  const int32_t* src;
  int32_t n_words, slot_word, lens_word;
  void* out;
  const void* q;
  void* k_cache;
  void* v_cache;
  int32_t* tables;
  int32_t max_blocks, num_blocks, S, H_q, H_kv, max_context_len;
  float sm_scale, k_scale, v_scale;
  const void* k_new;
  const void* v_new;
  int32_t* counters;
  float* partials;
};

template <typename CacheT, int D>
static pa_status launch_step(hipStream_t st, const StepArgs& a) {
  const int32_t shift = decode_chunk_shift(a.S, a.H_kv, a.max_context_len);
  const int32_t n_chunks = decode_num_chunks(a.max_context_len, shift);
  float* ws_ml = a.partials;
  float* ws_o = ws_ml + static_cast<int64_t>(a.S) * a.H_q * n_chunks * 2;
  const bool fp8 = sizeof(typename CacheT::raw) == 1;
  const float score_scale = a.sm_scale * kLog2e * (fp8 ? a.k_scale : 1.f);
  const float out_scale = fp8 ? a.v_scale : 1.f;
  // one fp32 reciprocal each, as the cache-write kernels use
  const float k_inv = fp8 ? 1.0f / a.k_scale : 1.f;
  const float v_inv = fp8 ? 1.0f / a.v_scale : 1.f;
  hipError_t e = launch(kDecodeStep, decode_step_kernel<CacheT, D>,
                        dim3(step_work_groups<CacheT, D>()), dim3(kThreads), 0, st, a.dst, a.src,
                        a.n_words, a.slot_word, a.lens_word,
                        g_step_spins.load(std::memory_order_relaxed),
                        static_cast<uint16_t*>(a.out),
                        static_cast<const uint16_t*>(a.q),
                        static_cast<typename CacheT::raw*>(a.k_cache),
                        static_cast<typename CacheT::raw*>(a.v_cache), a.tables, a.max_blocks,
                        a.num_blocks, a.S, a.H_q, a.H_kv, a.H_q / a.H_kv, n_chunks, shift,
                        score_scale, out_scale, static_cast<const uint16_t*>(a.k_new),
                        static_cast<const uint16_t*>(a.v_new), k_inv, v_inv, a.counters, ws_ml,
                        ws_o);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_decode_step: launch failed: %s", hipGetErrorString(e));
  if (n_chunks > 1)
    return launch_decode_merge(st, a.out, ws_ml, ws_o, a.dst + a.lens_word, a.max_blocks, kBlock,
                               a.S, a.H_q, D, n_chunks, shift, out_scale);
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_decode_step(void* stream, int32_t* dst, const void* src_host,
                                    size_t bytes, size_t slot_offset, size_t lens_offset,
                                    const void* k_new, const void* v_new, pa_dtype new_dt,
                                    void* out, pa_dtype out_dt, const void* q, pa_dtype q_dt,
                                    void* k_cache, void* v_cache, pa_dtype cache_dt,
                                    int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
                                    int32_t S, int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                                    int32_t max_context_len, float sm_scale, float k_scale,
                                    float v_scale, void* ws, size_t ws_bytes) {
  const char* who = "pa_decode_step";
  if (bs != kBlock) return fail(PA_ERR_INVALID, "%s: block size %d != 16", who, bs);
  if (S < 0 || S > kStepMaxSeqs || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 ||
      H_q / H_kv > kMaxGroup || H_kv > 65535)
    return fail(PA_ERR_INVALID,
                "%s: S=%d (at most %d), H_q=%d, H_kv=%d (at most %d query heads per KV head)",
                who, S, kStepMaxSeqs, H_q, H_kv, kMaxGroup);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "%s: D=%d not in {64,128}", who, D);
  if (q_dt != PA_BF16 || out_dt != PA_BF16 || new_dt != PA_BF16 ||
      (cache_dt != PA_BF16 && cache_dt != PA_FP8_E4M3))
    return fail(PA_ERR_INVALID,
                "%s: bf16 queries, outputs and new K/V with a bf16 or fp8 cache only "
                "(q=%d out=%d new=%d cache=%d)", who, q_dt, out_dt, new_dt, cache_dt);
  if (max_blocks <= 0 || num_blocks <= 0 || max_context_len <= 0)
    return fail(PA_ERR_INVALID, "%s: max_blocks=%d num_blocks=%d max_context_len=%d", who,
                max_blocks, num_blocks, max_context_len);
  if (static_cast<int64_t>(max_blocks) * kBlock > INT32_MAX ||
      static_cast<int64_t>(num_blocks) * kBlock > INT32_MAX)
    return fail(PA_ERR_INVALID, "%s: max_blocks=%d or num_blocks=%d too large", who, max_blocks,
                num_blocks);
  if (cache_dt == PA_FP8_E4M3 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
       !__builtin_isfinite(v_scale)))
    return fail(PA_ERR_INVALID, "%s: fp8 scales must be finite and > 0", who);
  if (!(sm_scale > 0.f) || !__builtin_isfinite(sm_scale))
    return fail(PA_ERR_INVALID, "%s: sm_scale must be finite and > 0", who);
  if (bytes % 4 != 0 || slot_offset % 4 != 0 || lens_offset % 4 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 4 != 0 || reinterpret_cast<uintptr_t>(src_host) % 4 != 0)
    return fail(PA_ERR_INVALID,
                "%s: bytes=%zu, the offsets (%zu, %zu) and both addresses must be multiples of 4",
                who, bytes, slot_offset, lens_offset);
  if (bytes / 4 > INT32_MAX) return fail(PA_ERR_INVALID, "%s: bytes=%zu too large", who, bytes);
  const size_t n = static_cast<size_t>(S);
  if (n > 0 && (slot_offset > bytes || (bytes - slot_offset) / 4 < n || lens_offset > bytes ||
                (bytes - lens_offset) / 4 < n))
    return fail(PA_ERR_INVALID,
                "%s: %d slots at byte %zu and %d lengths at byte %zu do not fit the %zu-byte "
                "buffer", who, S, slot_offset, S, lens_offset, bytes);
  if (S == 0) return PA_OK;
  if (!dst || !out || !q || !k_cache || !v_cache || !block_tables || !k_new || !v_new)
    return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  const size_t need = pa_decode_workspace_bytes(S, H_q, H_kv, D, max_context_len);
  if (!ws || ws_bytes < need)
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu required", who, ws_bytes, need);
  StepArgs a;
  a.dst = dst;
  a.src = nullptr;
  if (src_host) {
    void* src_dev = nullptr;
    const pa_status ps = pinned_alias(who, src_host, &src_dev);
    if (ps != PA_OK) return ps;
    a.src = static_cast<const int32_t*>(src_dev);
  }
  a.n_words = static_cast<int32_t>(bytes / 4);
  a.slot_word = static_cast<int32_t>(slot_offset / 4);
  a.lens_word = static_cast<int32_t>(lens_offset / 4);
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.S = S;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.max_context_len = max_context_len;
  a.sm_scale = sm_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.counters = static_cast<int32_t*>(ws);
  // the partials follow the counter region, as in pa_decode's workspace
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + decode_counter_bytes(S));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cache_dt == PA_BF16)
    return D == 128 ? launch_step<BF16, 128>(st, a) : launch_step<BF16, 64>(st, a);
  return D == 128 ? launch_step<FP8, 128>(st, a) : launch_step<FP8, 64>(st, a);
}

extern "C" pa_status pa_decode_step_set_spin_limit(int32_t polls) {
  if (polls < 1) return fail(PA_ERR_INVALID, "pa_decode_step_set_spin_limit: polls=%d < 1", polls);
  g_step_spins.store(polls, std::memory_order_relaxed);
  return PA_OK;
}
