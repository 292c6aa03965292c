// pa_prefill_chunk: causal attention of prefill slices against their paged
// prefix.
//
// LESSON "vLLM Serving Internals", "Chunked prefill": a long prompt is split
// into fixed-size slices (512 tokens by default), each scheduled as a unit;
// a slice's queries attend every earlier position of the prompt and the
// slice's own positions up to and including their own (causal).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

pa_status launch_attend_generic(hipStream_t st, void* out, pa_dtype out_dt, const void* q,
                                pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                                int32_t num_blocks, const int32_t* context_lens,
                                const int32_t* cu_q_lens, const int32_t* start_pos,
                                int32_t n_chunks, int32_t rows, int32_t H_q, int32_t H_kv,
                                int32_t D, float sm_scale, float k_scale, float v_scale);

}  // namespace pa

using namespace pa;

extern "C" size_t pa_prefill_workspace_bytes(int32_t n_chunks, int32_t max_q_len, int32_t H_q,
                                             int32_t H_kv, int32_t D, int32_t max_context_len) {
  (void)n_chunks;
  (void)max_q_len;
  (void)H_q;
  (void)H_kv;
  (void)D;
  (void)max_context_len;
  return 0;
}

extern "C" pa_status pa_prefill_chunk(void* stream, void* out, pa_dtype out_dt, const void* q,
                                      pa_dtype q_dt, const int32_t* cu_q_lens,
                                      const int32_t* start_pos, const void* k_cache,
                                      const void* v_cache, pa_dtype cache_dt,
                                      const int32_t* block_tables, int32_t max_blocks,
                                      int32_t num_blocks, int32_t n_chunks, int32_t H_q,
                                      int32_t H_kv, int32_t D, int32_t bs, int32_t max_q_len,
                                      int32_t max_context_len, float sm_scale, float k_scale,
                                      float v_scale, void* ws, size_t ws_bytes) {
  (void)ws;
  (void)ws_bytes;
  (void)max_context_len;
  if (bs != kBlock) return fail(PA_ERR_INVALID, "pa_prefill_chunk: block size %d != 16", bs);
  if (n_chunks < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: n_chunks=%d H_q=%d H_kv=%d", n_chunks, H_q,
                H_kv);
  if (D != 64 && D != 128)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: D=%d not in {64,128}", D);
  if (max_blocks <= 0 || num_blocks <= 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: max_blocks=%d num_blocks=%d max_q_len=%d",
                max_blocks, num_blocks, max_q_len);
  const bool f32 = q_dt == PA_F32 && cache_dt == PA_F32 && out_dt == PA_F32;
  const bool bf = q_dt == PA_BF16 && out_dt == PA_BF16 &&
                  (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3);
  if (!f32 && !bf)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: unsupported dtypes q=%d cache=%d out=%d",
                q_dt, cache_dt, out_dt);
  if (cache_dt == PA_FP8_E4M3 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
       !__builtin_isfinite(v_scale)))
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: fp8 scales must be finite and > 0");
  if (n_chunks == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !cu_q_lens || !start_pos || !k_cache || !v_cache || !block_tables)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: NULL buffer");
  if (static_cast<int64_t>(n_chunks) * max_q_len > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: too many query rows");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // slice lengths live on the device: launch max_q_len rows per slice and let
  // the rows past each slice's end exit
  return launch_attend_generic(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt, block_tables,
                               max_blocks, num_blocks, nullptr, cu_q_lens, start_pos, n_chunks,
                               max_q_len, H_q, H_kv, D, sm_scale, k_scale, v_scale);
}
