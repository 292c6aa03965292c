// pa_prefill_chunk: causal attention of prefill slices against their paged
// prefix.
//
// LESSON "vLLM Serving Internals", "Chunked prefill": a long prompt is split
// into fixed-size slices (512 tokens by default), each scheduled as a unit;
// a slice's queries attend every earlier position of the prompt and the
// slice's own positions up to and including their own (causal).  The keys
// and values of the prefix and of the slice itself are read from the paged
// cache through the sequence's block table ("vLLM architecture", section
// 2.3: compute within a block, accumulate across blocks), so the slice's own
// K/V are written with pa_cache_write first.
//
// bf16 queries with a bf16 or fp8 e4m3fn cache run on the matrix cores; an
// fp32 problem runs on the generic VALU kernel.  Q K^T multiplies bf16 by
// bf16 (v_mfma_f32_32x32x16_bf16).  P V multiplies fp16 by fp16
// (v_mfma_f32_32x32x16_f16): the softmax weights (a lane's 32 weights of a
// tile sum to at most kPfSafe = 2^15 before the reference is raised, so each
// stays finite in fp16) keep 11 significant bits in fp16 against 8 in bf16,
// which is what keeps a slice whose first rows see only a handful of keys
// within the output tolerance; V is converted to fp16 on its way into LDS (exact for e4m3 codes and for
// bf16 magnitudes up to 65504, larger bf16 values saturate).
//
// Work decomposition.  A work-group owns one KV head, up to eight of the
// query heads that share it (one wave each) and 32 consecutive query
// positions per wave; when a KV head has fewer than eight query heads the
// spare waves take further 32-position sub-tiles, so every wave of the group
// consumes the same K/V tile.  K/V arrive in tiles of 64 keys (four cache
// blocks), staged through four LDS stages: the global loads of a tile are
// issued two iterations before its keys are multiplied, so their latency
// hides behind a whole iteration of matrix work.  Inside each wave the
// tiles run as a software pipeline (see the main loop): the MFMAs of one
// tile's scores and of an older tile's P V product interleave with the
// exponentials of the tile in between, so that the matrix core and the
// vector unit work at once.  When the slices alone give too few work-groups
// to fill the chip, the key range is split and a second kernel merges the
// partial softmax states.
//
// Per wave and 32-key half-tile the scores are computed transposed,
// S^T = K Q^T (keys on the MFMA rows, the wave's 32 queries on its columns),
// so that a lane holds 16 scores of a single query.  The accumulator O^T =
// V^T P^T keeps the same orientation: each lane owns one query's column of
// O^T, so the softmax statistics and the rescaling never leave the lane
// except for one exchange with the lane 32 away that holds the query's other
// 16 keys.  The K rows of a 16-key group are stored in LDS with their middle
// quads swapped; with that permutation the 8 keys a lane holds for each
// 16-key step of P^T are consecutive, which is what one 16-byte read of the
// token-minor V layout supplies.
#include "pa_prefill_body.h"

namespace pa {

pa_status launch_attend_generic(hipStream_t st, void* out, pa_dtype out_dt, const void* q,
                                pa_dtype q_dt, const void* k_cache, const void* v_cache,
                                pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                                int32_t num_blocks, const int32_t* context_lens,
                                const int32_t* cu_q_lens, const int32_t* start_pos,
                                int32_t n_chunks, int32_t rows, int32_t H_q, int32_t H_kv,
                                int32_t D, float sm_scale, float k_scale, float v_scale);

namespace {

// grid.x = H_kv * n_head_groups * n_split * n_pos_tiles (KV head fastest, so
// the groups sharing a KV head land on the same XCD's L2); grid.y = slices.
template <typename CacheT, int D, int BS>
__global__ __launch_bounds__(kPfThreads) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ start_pos,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, int32_t num_blocks, int32_t H_q, PfGeom geo, float score_scale,
    float v_scale, float* __restrict__ ws_ml, uint16_t* __restrict__ ws_o, int32_t ws_rows) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * stage_bytes<D>()];
  prefill_block<CacheT, D, false, BS>(smem, blockIdx.x, blockIdx.y, out, q, cu_q_lens, start_pos,
                                  k_cache, v_cache, block_tables, max_blocks, num_blocks, H_q, geo,
                                  score_scale, v_scale, ws_ml, ws_o, ws_rows, nullptr);
}

// Merge the key-range partials of each (row, head): D/4 threads per pair,
// four dimensions each.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    uint16_t* __restrict__ out, const int32_t* __restrict__ cu_q_lens, int32_t n_chunks,
    int32_t H_q, int32_t n_split, const float* __restrict__ ws_ml,
    const uint16_t* __restrict__ ws_o, int32_t ws_rows, float v_scale) {
  constexpr int T = D / 4;
  const int sub = threadIdx.x % T;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (256 / T) + threadIdx.x / T;
  const int64_t total =
      min(static_cast<int64_t>(cu_q_lens[n_chunks]), static_cast<int64_t>(ws_rows)) * H_q;
  if (pair >= total) return;
  const int64_t stride = static_cast<int64_t>(ws_rows) * H_q;
  const float M = pf_merge_max(ws_ml, pair, stride, n_split);
  const float inv = pf_merge_inv(ws_ml, pair, stride, n_split, M, v_scale);
  const f32x4 acc = pf_merge_dims4<D>(ws_ml, ws_o, pair, stride, n_split, M, 4 * sub);
  *reinterpret_cast<u32x2*>(out + pair * D + 4 * sub) = pack_bf16x4(acc, inv);
}

template <typename CacheT, int D, int BS>
pa_status launch_prefill_mfma(hipStream_t st, void* out, const void* q, const int32_t* cu_q_lens,
                              const int32_t* start_pos, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
                              int32_t n_chunks, int32_t H_q, int32_t H_kv, int32_t max_q_len,
                              int32_t max_context_len, float score_scale, float v_scale, void* ws,
                              size_t ws_bytes) {
  const PfGeom geo = pf_geometry(n_chunks, max_q_len, H_q, H_kv, max_context_len);
  const int64_t gx = static_cast<int64_t>(H_kv) * geo.n_head_groups * geo.n_split * geo.n_pos_tiles;
  if (gx > INT32_MAX || n_chunks > 65535)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: grid too large (%lld x %d)",
                static_cast<long long>(gx), n_chunks);
  const int32_t ws_rows = n_chunks * max_q_len;
  float* ws_ml = nullptr;
  uint16_t* ws_o = nullptr;
  if (geo.n_split > 1) {
    // [normalised partial outputs, fp16][partial (m, l), fp32]
    const size_t need = static_cast<size_t>(geo.n_split) * ws_rows * H_q * pf_slot_bytes(D);
    if (!ws || ws_bytes < need)
      return fail(PA_ERR_WORKSPACE, "pa_prefill_chunk: workspace %zu bytes < %zu", ws_bytes, need);
    ws_o = static_cast<uint16_t*>(ws);
    ws_ml = reinterpret_cast<float*>(ws_o + static_cast<size_t>(geo.n_split) * ws_rows * H_q * D);
  }
  hipError_t e = launch(kPrefill, prefill_kernel<CacheT, D, BS>,
                        dim3(static_cast<uint32_t>(gx), n_chunks), dim3(kPfThreads), 0, st,
                        static_cast<uint16_t*>(out),
                        static_cast<const uint16_t*>(q), cu_q_lens, start_pos,
                        static_cast<const typename CacheT::raw*>(k_cache),
                        static_cast<const typename CacheT::raw*>(v_cache), block_tables, max_blocks,
                        num_blocks, H_q, geo, score_scale, v_scale, ws_ml, ws_o, ws_rows);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_prefill_chunk: launch failed: %s", hipGetErrorString(e));
  if (geo.n_split > 1) {
    const int64_t pairs = static_cast<int64_t>(ws_rows) * H_q;
    constexpr int kPairsPerGroup = 256 / (D / 4);
    e = launch(kPrefillMerge, prefill_merge_kernel<D>,
               dim3(static_cast<uint32_t>((pairs + kPairsPerGroup - 1) / kPairsPerGroup)),
               dim3(256), 0, st, static_cast<uint16_t*>(out), cu_q_lens, n_chunks, H_q,
               geo.n_split, ws_ml, ws_o, ws_rows, v_scale);
    if (e != hipSuccess)
      return fail(PA_ERR_DEVICE, "pa_prefill_chunk: merge launch failed: %s",
                  hipGetErrorString(e));
  }
  return PA_OK;
}

bool prefill_uses_mfma(pa_dtype q_dt, pa_dtype cache_dt) {
  return q_dt == PA_BF16 && (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" size_t pa_prefill_workspace_bytes(int32_t n_chunks, int32_t max_q_len, int32_t H_q,
                                             int32_t H_kv, int32_t D, int32_t max_context_len) {
  if (n_chunks <= 0 || max_q_len <= 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 ||
      (D != 64 && D != 128))
    return 0;
  return pf_partials_bound(n_chunks, max_q_len, H_q, H_kv, D, max_context_len);
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
  if (bs != 8 && bs != 16 && bs != 32)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: block size %d not in {8, 16, 32}", bs);
  if (n_chunks < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: n_chunks=%d H_q=%d H_kv=%d", n_chunks, H_q,
                H_kv);
  if (D != 64 && D != 128)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: D=%d not in {64,128}", D);
  if (max_blocks <= 0 || num_blocks <= 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: max_blocks=%d num_blocks=%d max_q_len=%d",
                max_blocks, num_blocks, max_q_len);
  if (max_context_len < max_q_len ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(bs) * max_blocks)
    return fail(PA_ERR_INVALID,
                "pa_prefill_chunk: max_context_len=%d must lie in [max_q_len=%d, bs*max_blocks=%lld]",
                max_context_len, max_q_len, static_cast<long long>(bs) * max_blocks);
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
  if (!(sm_scale > 0.f) || !__builtin_isfinite(sm_scale))
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: sm_scale must be finite and > 0");
  if (n_chunks == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !cu_q_lens || !start_pos || !k_cache || !v_cache || !block_tables)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: NULL buffer");
  if (static_cast<int64_t>(n_chunks) * max_q_len > INT32_MAX / 64)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: too many query rows");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!prefill_uses_mfma(q_dt, cache_dt) && bs != kBlock)
    return fail(PA_ERR_INVALID,
                "pa_prefill_chunk: block size %d needs the matrix-core path (bf16 queries, bf16 or "
                "fp8 cache)", bs);
  if (!prefill_uses_mfma(q_dt, cache_dt)) {
    // slice lengths live on the device: launch max_q_len rows per slice and
    // let the rows past each slice's end exit
    return launch_attend_generic(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt,
                                 block_tables, max_blocks, num_blocks, nullptr, cu_q_lens,
                                 start_pos, n_chunks, max_q_len, H_q, H_kv, D, sm_scale, k_scale,
                                 v_scale);
  }
  // log2-domain score scale; fp8 keys carry k_scale, values v_scale
  const float kscale = cache_dt == PA_FP8_E4M3 ? k_scale : 1.f;
  const float vscale = cache_dt == PA_FP8_E4M3 ? v_scale : 1.f;
  const float score_scale = sm_scale * kscale * kLog2e;
  auto run = [&](auto cache_tag, auto d_tag, auto bs_tag) {
    using C = decltype(cache_tag);
    return launch_prefill_mfma<C, decltype(d_tag)::value, decltype(bs_tag)::value>(
        st, out, q, cu_q_lens, start_pos, k_cache, v_cache, block_tables, max_blocks, num_blocks,
        n_chunks, H_q, H_kv, max_q_len, max_context_len, score_scale, vscale, ws, ws_bytes);
  };
  auto by_bs = [&](auto cache_tag, auto d_tag) {
    if (bs == 8) return run(cache_tag, d_tag, std::integral_constant<int, 8>{});
    if (bs == 32) return run(cache_tag, d_tag, std::integral_constant<int, 32>{});
    return run(cache_tag, d_tag, std::integral_constant<int, 16>{});
  };
  auto by_d = [&](auto cache_tag) {
    if (D == 128) return by_bs(cache_tag, std::integral_constant<int, 128>{});
    return by_bs(cache_tag, std::integral_constant<int, 64>{});
  };
  if (cache_dt == PA_BF16) return by_d(BF16{});
  return by_d(FP8{});
}
