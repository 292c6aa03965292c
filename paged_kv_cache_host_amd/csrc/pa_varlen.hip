// pa_attend_varlen: the attention of one continuous-batching iteration --
// its decode rows and its prefill slices -- in a single kernel launch.
//
// LESSON "vLLM Serving Internals", "What the scheduler looks like": each
// iteration runs the whole mixed batch (decode tokens of running sequences
// plus chunked-prefill slices) as one forward call on the GPU; "Chunked
// prefill": a slice attends causally to its prompt's earlier positions and
// its own.  A decode row is a sequence with one new query; a prefill slice
// is a sequence with up to max_q_len new queries.  Both read their K/V from
// the paged cache through their block-table row (ARTICLE 2.3).
//
// One persistent launch of work-groups with the prefill work-group's shape
// (8 waves, one work-group per compute unit by LDS):
//   - work-groups 0 .. pf_items-1 first run one prefill item each, the same
//     item (slice, KV head, head group, key-range split, position tile) and
//     the same XCD as work-group x of slice c in the prefill launch, so the
//     work-groups that share a KV head still share an L2;
//   - then every work-group, and pf_items .. grid-1 straight away, takes
//     decode items (sequence, KV head, chunk) from the decode ticket queue
//     until it is empty.
// The long prefill items are dispatched first and the short decode items
// fill the compute units as prefill items end, so the launch has one tail
// rather than one per kernel.  Key-range splits of a prefill group and the
// chunks of a long decode context are merged inside the launch by the last
// of their work-groups to finish (the same arithmetic as the separate merge
// kernels, so results match the separate launches bit for bit when the
// split choices agree).  LDS is shared: a work-group's prefill stages and
// its decode lists are never live at once.
#include "pa_decode_body.h"
#include "pa_prefill_body.h"

#include <algorithm>
#include <type_traits>

namespace pa {
namespace {

template <int D>
constexpr size_t varlen_lds_bytes() {
  return std::max<size_t>(4 * stage_bytes<D>(), sizeof(DecodeShared<D>));
}

static_assert(kThreads == kPfThreads, "decode and prefill work-groups have one shape");

template <typename CacheT, int D>
__global__ __launch_bounds__(kThreads) void varlen_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ seq_lens,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ dec_tables,
    int32_t dec_max_blocks, const int32_t* __restrict__ pf_tables, int32_t pf_max_blocks,
    int32_t num_blocks, int32_t n_decode, int32_t H_q, int32_t H_kv,
    PfGeom geo, int32_t pf_gx, int32_t pf_items, float* __restrict__ pf_ws_ml,
    uint16_t* __restrict__ pf_ws_o, int32_t pf_ws_rows, int32_t dec_chunks, int32_t dec_shift,
    float* __restrict__ dec_ws_ml, float* __restrict__ dec_ws_o, float score_scale,
    float v_scale, int32_t* __restrict__ counters, int32_t* __restrict__ dec_merge,
    int32_t* __restrict__ pf_merge) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[varlen_lds_bytes<D>()];
  const int32_t b = blockIdx.x;
  if (b < pf_items) {
    prefill_block<CacheT, D, true, kBlock>(
        lds, b % pf_gx, b / pf_gx, out, q, cu_q_lens + n_decode, seq_lens + n_decode, k_cache,
        v_cache, pf_tables, pf_max_blocks, num_blocks, H_q, geo, score_scale, v_scale, pf_ws_ml,
        pf_ws_o, pf_ws_rows, pf_merge);
    __syncthreads();  // the stages are done before the decode lists reuse them
  }
  decode_work<CacheT, D, kBlock, true>(*reinterpret_cast<DecodeShared<D>*>(lds), out, q, k_cache,
                                       v_cache, dec_tables, dec_max_blocks, num_blocks, seq_lens,
                                       n_decode, H_q, H_kv, H_q / H_kv, dec_chunks, dec_shift,
                                       score_scale, v_scale, counters, dec_ws_ml, dec_ws_o,
                                       dec_merge);
  decode_finish(counters);
}

// Everything a call needs to know about its launch, from host-side bounds
// only (the lengths themselves stay on the device).
struct VarlenPlan {
  PfGeom geo;
  int64_t pf_gx = 0, pf_items = 0, pf_groups = 0;  // groups: merge counters
  int32_t pf_ws_rows = 0;
  int32_t dec_shift = 0, dec_chunks = 1;
  int64_t n_counters = 2;   // ticket, done, then the merge counters
  size_t dec_bytes = 0, pf_bytes = 0;
};

VarlenPlan varlen_plan(int32_t n_decode, int32_t n_prefill, int32_t H_q, int32_t H_kv, int32_t D,
                       int32_t max_q_len, int32_t max_decode_len, int32_t max_prefill_len) {
  VarlenPlan p;
  if (n_prefill > 0 && max_q_len > 0) {
    p.geo = pf_geometry(n_prefill, max_q_len, H_q, H_kv, max_prefill_len);
    p.pf_gx = static_cast<int64_t>(H_kv) * p.geo.n_head_groups * p.geo.n_split *
              p.geo.n_pos_tiles;
    p.pf_items = p.pf_gx * n_prefill;
    p.pf_groups = p.pf_items / p.geo.n_split;
    p.pf_ws_rows = n_prefill * max_q_len;
    if (p.geo.n_split > 1)
      p.pf_bytes = static_cast<size_t>(p.geo.n_split) * p.pf_ws_rows * H_q * pf_slot_bytes(D);
  } else {
    p.geo = PfGeom{H_kv, H_q / H_kv, 1, 1, 1, 0, 1};
  }
  if (n_decode > 0) {
    p.dec_shift = decode_chunk_shift(n_decode, H_kv, max_decode_len);
    p.dec_chunks = decode_num_chunks(max_decode_len, p.dec_shift);
    if (p.dec_chunks > 1)
      p.dec_bytes = (static_cast<size_t>(n_decode) * H_q * p.dec_chunks * (D + 2) * sizeof(float) +
                     255) &
                    ~static_cast<size_t>(255);
  }
  p.n_counters = 2 + static_cast<int64_t>(n_decode) * H_kv + p.pf_groups;
  return p;
}

// Compute units of the current device (cached per device).
int32_t device_cus() {
  static int32_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev] = cus;
  return cus;
}

template <typename CacheT, int D>
pa_status launch_varlen(hipStream_t st, const VarlenPlan& p, void* out, const void* q,
                        const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t n_decode,
                        const void* k_cache, const void* v_cache, const int32_t* dec_tables,
                        int32_t dec_max_blocks, const int32_t* pf_tables, int32_t pf_max_blocks,
                        int32_t num_blocks, int32_t H_q, int32_t H_kv, float score_scale,
                        float v_scale, int32_t* counters, void* ws) {
  int32_t* dec_merge = counters + 2;
  int32_t* pf_merge = dec_merge + static_cast<int64_t>(n_decode) * H_kv;
  char* base = static_cast<char*>(ws);
  float* dec_ws_ml = reinterpret_cast<float*>(base);
  float* dec_ws_o = dec_ws_ml + static_cast<int64_t>(n_decode) * H_q * p.dec_chunks * 2;
  uint16_t* pf_ws_o = reinterpret_cast<uint16_t*>(base + p.dec_bytes);
  float* pf_ws_ml = reinterpret_cast<float*>(
      pf_ws_o + static_cast<int64_t>(p.geo.n_split) * p.pf_ws_rows * H_q * D);
  // decode-only work-groups: one per compute unit (the kernel's LDS admits
  // one work-group per unit), none when there are no decode rows
  const int64_t grid = p.pf_items + (n_decode > 0 ? device_cus() : 0);
  const hipError_t e =
      launch(kVarlen, varlen_kernel<CacheT, D>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads),
             0, st, static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q), cu_q_lens,
             seq_lens, static_cast<const typename CacheT::raw*>(k_cache),
             static_cast<const typename CacheT::raw*>(v_cache), dec_tables, dec_max_blocks,
             pf_tables, pf_max_blocks, num_blocks, n_decode, H_q, H_kv, p.geo,
             static_cast<int32_t>(p.pf_gx),
             static_cast<int32_t>(p.pf_items), pf_ws_ml, pf_ws_o, p.pf_ws_rows, p.dec_chunks,
             p.dec_shift, dec_ws_ml, dec_ws_o, score_scale, v_scale, counters, dec_merge,
             pf_merge);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_attend_varlen: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int64_t pa_attend_varlen_counters(int32_t n_decode, int32_t n_prefill, int32_t H_q,
                                             int32_t H_kv, int32_t max_q_len) {
  if (n_decode < 0 || n_prefill < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 || max_q_len < 0)
    return 0;
  // the merge counters depend on neither D nor the context bounds
  return varlen_plan(n_decode, n_prefill, H_q, H_kv, 64, max_q_len, 1, 1).n_counters;
}

extern "C" size_t pa_attend_varlen_workspace_bytes(int32_t n_decode, int32_t n_prefill,
                                                   int32_t H_q, int32_t H_kv, int32_t D,
                                                   int32_t max_q_len, int32_t max_decode_len,
                                                   int32_t max_prefill_len) {
  if (n_decode < 0 || n_prefill < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 ||
      (D != 64 && D != 128) || max_q_len < 0 || max_decode_len < 0 || max_prefill_len < 0)
    return 0;
  // an upper bound over every call with at most these sizes: the decode
  // partials for the smallest chunk size, the prefill partials for the
  // largest split any smaller batch can get
  size_t dec = 0;
  if (n_decode > 0)
    dec = (static_cast<size_t>(n_decode) * H_q *
               decode_num_chunks(max_decode_len, kMinChunkShift) * (D + 2) * sizeof(float) +
           255) &
          ~static_cast<size_t>(255);
  const size_t pf = n_prefill > 0 && max_q_len > 0
                        ? pf_partials_bound(n_prefill, max_q_len, H_q, H_kv, D, max_prefill_len)
                        : 0;
  return dec + pf;
}

extern "C" pa_status pa_attend_varlen(void* stream, void* out, pa_dtype out_dt, const void* q,
                                      pa_dtype q_dt, const int32_t* cu_q_lens,
                                      const int32_t* seq_lens, int32_t n_decode,
                                      int32_t n_prefill, const void* k_cache, const void* v_cache,
                                      pa_dtype cache_dt, const int32_t* dec_tables,
                                      int32_t dec_max_blocks, const int32_t* pf_tables,
                                      int32_t pf_max_blocks, int32_t num_blocks, int32_t H_q,
                                      int32_t H_kv, int32_t D, int32_t bs, int32_t max_q_len,
                                      int32_t max_decode_len, int32_t max_prefill_len,
                                      float sm_scale, float k_scale, float v_scale,
                                      int32_t* counters, int64_t n_counters, void* ws,
                                      size_t ws_bytes) {
  const char* who = "pa_attend_varlen";
  if (bs != kBlock) return fail(PA_ERR_INVALID, "%s: block size %d != 16", who, bs);
  if (n_decode < 0 || n_prefill < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return fail(PA_ERR_INVALID, "%s: n_decode=%d n_prefill=%d H_q=%d H_kv=%d", who, n_decode,
                n_prefill, H_q, H_kv);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "%s: D=%d not in {64,128}", who, D);
  if (!(q_dt == PA_BF16 && out_dt == PA_BF16 &&
        (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3)))
    return fail(PA_ERR_INVALID,
                "%s: the fused launch takes bf16 queries and outputs with a bf16 or fp8 cache "
                "(q=%d cache=%d out=%d); other types go through pa_decode and pa_prefill_chunk",
                who, q_dt, cache_dt, out_dt);
  if (H_q / H_kv > kMaxGroup)
    return fail(PA_ERR_INVALID, "%s: %d query heads per KV head exceed %d", who, H_q / H_kv,
                kMaxGroup);
  if (num_blocks <= 0 || max_q_len < 0 || max_decode_len < 0 || max_prefill_len < 0 ||
      (n_decode > 0 && dec_max_blocks <= 0) || (n_prefill > 0 && pf_max_blocks <= 0))
    return fail(PA_ERR_INVALID,
                "%s: dec_max_blocks=%d pf_max_blocks=%d num_blocks=%d max_q_len=%d "
                "max_decode_len=%d max_prefill_len=%d",
                who, dec_max_blocks, pf_max_blocks, num_blocks, max_q_len, max_decode_len,
                max_prefill_len);
  if ((n_decode > 0 && max_decode_len > 16LL * dec_max_blocks) ||
      (n_prefill > 0 && max_prefill_len > 16LL * pf_max_blocks) ||
      (n_prefill > 0 && max_prefill_len < max_q_len))
    return fail(PA_ERR_INVALID,
                "%s: max_decode_len=%d must lie within 16*dec_max_blocks=%lld, max_prefill_len=%d "
                "within 16*pf_max_blocks=%lld and >= max_q_len=%d",
                who, max_decode_len, 16LL * dec_max_blocks, max_prefill_len,
                16LL * pf_max_blocks, max_q_len);
  if (n_decode > kMaxSeqsPerLaunch)
    return fail(PA_ERR_INVALID, "%s: %d decode rows exceed %d per launch", who, n_decode,
                kMaxSeqsPerLaunch);
  if (cache_dt == PA_FP8_E4M3 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
       !__builtin_isfinite(v_scale)))
    return fail(PA_ERR_INVALID, "%s: fp8 scales must be finite and > 0", who);
  if (!(sm_scale > 0.f) || !__builtin_isfinite(sm_scale))
    return fail(PA_ERR_INVALID, "%s: sm_scale must be finite and > 0", who);
  if (n_prefill > 0 && max_q_len == 0) n_prefill = 0;  // every slice is empty
  if (n_decode == 0 && n_prefill == 0) return PA_OK;
  if (!out || !q || !cu_q_lens || !seq_lens || !k_cache || !v_cache ||
      (n_decode > 0 && !dec_tables) || (n_prefill > 0 && !pf_tables))
    return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  if (!counters) return fail(PA_ERR_WORKSPACE, "%s: NULL counters", who);
  if (static_cast<int64_t>(n_prefill) * max_q_len + n_decode > INT32_MAX / 64)
    return fail(PA_ERR_INVALID, "%s: too many query rows", who);
  const VarlenPlan p = varlen_plan(n_decode, n_prefill, H_q, H_kv, D, max_q_len, max_decode_len,
                                   max_prefill_len);
  if (p.pf_items + device_cus() > INT32_MAX)
    return fail(PA_ERR_INVALID, "%s: grid too large", who);
  if (n_counters < p.n_counters)
    return fail(PA_ERR_WORKSPACE, "%s: %lld counters < %lld required", who,
                static_cast<long long>(n_counters), static_cast<long long>(p.n_counters));
  const size_t need = p.dec_bytes + p.pf_bytes;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu required", who, ws_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // log2-domain score scale; fp8 keys carry k_scale, values v_scale
  const bool fp8 = cache_dt == PA_FP8_E4M3;
  const float score_scale = sm_scale * (fp8 ? k_scale : 1.f) * kLog2e;
  const float vscale = fp8 ? v_scale : 1.f;
  auto run = [&](auto cache_tag, auto d_tag) {
    return launch_varlen<decltype(cache_tag), decltype(d_tag)::value>(
        st, p, out, q, cu_q_lens, seq_lens, n_decode, k_cache, v_cache, dec_tables,
        dec_max_blocks, pf_tables, pf_max_blocks, num_blocks, H_q, H_kv, score_scale, vscale,
        counters, ws);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  if (!fp8) return D == 128 ? run(BF16{}, D128{}) : run(BF16{}, D64{});
  return D == 128 ? run(FP8{}, D128{}) : run(FP8{}, D64{});
}
