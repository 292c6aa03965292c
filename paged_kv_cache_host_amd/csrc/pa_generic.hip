// General attention kernel over the paged cache, on the vector ALUs.
//
// Serves every element type (fp32 caches and queries in particular) and the
// shapes outside the matrix-core kernels (more than 16 query heads per KV
// head).  One wave computes one (query row, query head): it walks the keys
// 0 .. limit-1 of the row's sequence 64 at a time (one key per lane), keeps
// an online softmax (ARTICLE "vLLM inference engine architecture" §2.3:
// scores within a block, accumulated across blocks), and accumulates the
// output with each lane owning D/64 dimensions.
//
// A row is either a decode query (row r of the batch, limit = context_lens[r],
// block-table row r) or a prefill-slice query (LESSON "vLLM Serving
// Internals", "Chunked prefill": query i of slice c at position
// start_pos[c] + i sees keys 0 .. start_pos[c] + i).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <typename T>
__device__ __forceinline__ float load_f(const typename T::raw* p, int64_t i) {
  if constexpr (sizeof(typename T::raw) == 4)
    return p[i];
  else if constexpr (sizeof(typename T::raw) == 2)
    return bf16_to_f32(p[i]);
  else
    return fp8_to_f32(p[i]);
}

template <typename QT, typename CacheT, typename OutT>
__global__ __launch_bounds__(kWave) void attend_generic_kernel(
    typename OutT::raw* __restrict__ out, const typename QT::raw* __restrict__ q,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, int32_t num_blocks, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ start_pos,
    int32_t H_q, int32_t H_kv, int32_t D, float score_scale, float out_scale) {
  __shared__ float q_s[128];
  __shared__ float p_s[kWave];
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  const int kvh = h / (H_q / H_kv);

  int64_t row, trow;
  int32_t limit;
  if (cu_q_lens == nullptr) {
    // decode: grid (S, H_q, 1)
    row = trow = blockIdx.x;
    limit = context_lens[row];
  } else {
    // prefill slice c = blockIdx.z, query i = blockIdx.x of that slice
    const int c = blockIdx.z;
    const int32_t i = blockIdx.x;
    const int32_t q0 = cu_q_lens[c];
    if (i >= cu_q_lens[c + 1] - q0) return;
    row = q0 + i;
    trow = c;
    limit = start_pos[c] + i + 1;
  }
  limit = min(limit, max_blocks * kBlock);
  const int32_t* table = block_tables + trow * max_blocks;

  for (int d = lane; d < D; d += kWave) q_s[d] = load_f<QT>(q, (row * H_q + h) * D + d);
  __syncthreads();

  float m_run = -__builtin_inff(), l_run = 0.f;
  float acc[2] = {0.f, 0.f};
  for (int32_t k0 = 0; k0 < limit; k0 += kWave) {
    const int32_t key = k0 + lane;
    float s = -__builtin_inff();
    if (key < limit) {
      const int64_t tile =
          static_cast<int64_t>(safe_block(table[key / kBlock], num_blocks)) * H_kv + kvh;
      // K tile layout [D/X][16][X]: dim d of token o at (d/X)*16*X + o*X + d%X
      constexpr int X = 16 / sizeof(typename CacheT::raw);
      const int64_t kb = tile * kBlock * D + static_cast<int64_t>(key % kBlock) * X;
      float dot = 0.f;
      for (int d = 0; d < D; ++d)
        dot += q_s[d] * load_f<CacheT>(k_cache, kb + (d / X) * (kBlock * X) + d % X);
      s = dot * score_scale;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = __builtin_amdgcn_exp2f(s - m_new);
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    p_s[lane] = p;
    __syncthreads();
    const int32_t nk = min(kWave, limit - k0);
    for (int i = 0; i < 2; ++i) {
      const int d = lane + kWave * i;
      if (d >= D) break;
      float a = acc[i] * alpha;
      for (int j = 0; j < nk; ++j) {
        const int32_t kk = k0 + j;
        const int64_t tile =
            static_cast<int64_t>(safe_block(table[kk / kBlock], num_blocks)) * H_kv + kvh;
        a += p_s[j] * load_f<CacheT>(v_cache, tile * kBlock * D + static_cast<int64_t>(d) * kBlock +
                                                  kk % kBlock);
      }
      acc[i] = a;
    }
    __syncthreads();
  }
  const float inv = limit > 0 ? out_scale / l_run : 0.f;
  for (int i = 0; i < 2; ++i) {
    const int d = lane + kWave * i;
    if (d >= D) break;
    const float v = acc[i] * inv;
    if constexpr (sizeof(typename OutT::raw) == 2)
      out[(row * H_q + h) * D + d] = f32_to_bf16(v);
    else
      out[(row * H_q + h) * D + d] = v;
  }
}

template <typename QT, typename CacheT, typename OutT>
static pa_status launch_generic_t(hipStream_t st, void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks, int32_t num_blocks,
                                  const int32_t* context_lens, const int32_t* cu_q_lens,
                                  const int32_t* start_pos, int32_t n_chunks, int32_t rows,
                                  int32_t H_q, int32_t H_kv, int32_t D, float score_scale,
                                  float out_scale) {
  // decode: one row per sequence; prefill: rows = longest slice, one z per slice
  const dim3 grid(rows, H_q, cu_q_lens ? n_chunks : 1);
  hipError_t e = launch(kGeneric, attend_generic_kernel<QT, CacheT, OutT>, grid, dim3(kWave), 0, st,
                        static_cast<typename OutT::raw*>(out),
                        static_cast<const typename QT::raw*>(q),
                        static_cast<const typename CacheT::raw*>(k_cache),
                        static_cast<const typename CacheT::raw*>(v_cache), block_tables, max_blocks,
                        num_blocks, context_lens, cu_q_lens, start_pos, H_q, H_kv, D, score_scale,
                        out_scale);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "generic attention launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

pa_status launch_attend_generic(hipStream_t st, void* out, pa_dtype out_dt, const void* q,
                                pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                                int32_t num_blocks, const int32_t* context_lens,
                                const int32_t* cu_q_lens, const int32_t* start_pos,
                                int32_t n_chunks, int32_t rows, int32_t H_q, int32_t H_kv,
                                int32_t D, float sm_scale, float k_scale, float v_scale) {
  if (rows == 0) return PA_OK;
  if (H_q > 65535 || n_chunks > 65535)
    return fail(PA_ERR_INVALID, "H_q=%d or n_chunks=%d exceeds grid limits", H_q, n_chunks);
  if (q_dt == PA_F32 && cache_dt == PA_F32 && out_dt == PA_F32)
    return launch_generic_t<F32, F32, F32>(st, out, q, k_cache, v_cache, block_tables, max_blocks,
                                           num_blocks, context_lens, cu_q_lens, start_pos,
                                           n_chunks, rows, H_q, H_kv, D, sm_scale * kLog2e, 1.f);
  if (q_dt == PA_BF16 && cache_dt == PA_BF16 && out_dt == PA_BF16)
    return launch_generic_t<BF16, BF16, BF16>(st, out, q, k_cache, v_cache, block_tables,
                                              max_blocks, num_blocks, context_lens, cu_q_lens,
                                              start_pos, n_chunks, rows, H_q, H_kv, D,
                                              sm_scale * kLog2e, 1.f);
  if (q_dt == PA_BF16 && cache_dt == PA_FP8_E4M3 && out_dt == PA_BF16)
    return launch_generic_t<BF16, FP8, BF16>(st, out, q, k_cache, v_cache, block_tables,
                                             max_blocks, num_blocks, context_lens, cu_q_lens,
                                             start_pos, n_chunks, rows, H_q, H_kv, D,
                                             sm_scale * kLog2e * k_scale, v_scale);
  return fail(PA_ERR_INVALID, "unsupported dtypes q=%d cache=%d out=%d", q_dt, cache_dt, out_dt);
}

}  // namespace pa
