// pa_cache_write: scatter new K/V vectors into the paged cache.
//
// LESSON "vLLM Serving Internals", "The Concept: PagedAttention as a virtual
// memory system": the K/V of token position p of a sequence live in block
// table[p / bs] at offset p % bs.  The host turns positions into flat slots
// (block * bs + offset); this kernel stores each token's K and V at its slot
// for every KV head, optionally quantising bf16 to fp8 e4m3fn with a
// per-tensor scale.
//
// Layout per (block, KV head), x = elements per 16 bytes of the cache type:
//   K [D/x][16][x]   (16-byte chunks of the 16 tokens side by side)
//   V [D][16]        (a token's value is a column)
// One work-group takes 16 consecutive input tokens of one KV head.  K: each
// thread moves one (token, 16-byte chunk); V: the 16 x D tile is staged in
// LDS and written column-wise, so that when the 16 tokens fill one block in
// order (the prefill case) every write of a work-group is contiguous.
#include "pa_copy.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <typename NewT, typename CacheT>
__device__ __forceinline__ typename CacheT::raw encode(typename NewT::raw x, float inv_scale);

template <>
__device__ __forceinline__ float encode<F32, F32>(float x, float) {
  return x;
}
template <>
__device__ __forceinline__ uint16_t encode<BF16, BF16>(uint16_t x, float) {
  return x;
}
template <>
__device__ __forceinline__ uint8_t encode<BF16, FP8>(uint16_t x, float inv_scale) {
  return f32_to_e4m3_sat(bf16_to_f32(x) * inv_scale);
}

// One work-group's share: 16 consecutive input tokens (from t0 = 16 bx) of
// KV head h.  HOST_SLOTS: the slot mapping lies in pinned host memory and is
// read with system-scope loads (the fused staging kernel); otherwise it is
// device memory.
template <typename NewT, typename CacheT, int D, bool HOST_SLOTS, int BS>
__device__ __forceinline__ void cw_tile(int bx, int h, const typename NewT::raw* __restrict__ k_new,
                                        const typename NewT::raw* __restrict__ v_new,
                                        const int32_t* __restrict__ slots, int32_t n,
                                        typename CacheT::raw* __restrict__ k_cache,
                                        typename CacheT::raw* __restrict__ v_cache,
                                        int32_t num_blocks, int32_t H_kv, float k_inv,
                                        float v_inv) {
  using NR = typename NewT::raw;
  using CR = typename CacheT::raw;
  constexpr int X = 16 / sizeof(CR);  // cache elements per 16-byte chunk
  constexpr int NCH = D / X;          // chunks per token row
  __shared__ NR v_s[16][D + 2];
  __shared__ int32_t slot_s[16];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(bx) * 16;
  if (tid < 16) {
    const int64_t t = t0 + tid;
    int32_t sl = -1;
    if (t < n) {
      if constexpr (HOST_SLOTS)
        sl = __hip_atomic_load(slots + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else
        sl = slots[t];
    }
    if (sl >= num_blocks * BS) sl = -1;
    slot_s[tid] = sl;
  }
  // stage V rows of the 16 tokens
  for (int i = tid; i < 16 * D; i += 256) {
    const int tt = i / D, d = i % D;
    const int64_t t = t0 + tt;
    v_s[tt][d] = t < n ? v_new[(t * H_kv + h) * D + d] : NR(0);
  }
  __syncthreads();
  // K: thread -> (chunk, token)
  for (int i = tid; i < 16 * NCH; i += 256) {
    const int tt = i & 15, ch = i >> 4;
    const int32_t sl = slot_s[tt];
    if (sl < 0) continue;
    const int64_t t = t0 + tt;
    const int32_t blk = sl / BS, off = sl % BS;
    const NR* src = k_new + (t * H_kv + h) * D + ch * X;
    CR* dst = k_cache + ((static_cast<int64_t>(blk) * H_kv + h) * NCH + ch) * (BS * X) + off * X;
#pragma unroll
    for (int j = 0; j < X; ++j) dst[j] = encode<NewT, CacheT>(src[j], k_inv);
  }
  // V: thread -> (d, token), 16 adjacent threads share d
  for (int i = tid; i < 16 * D; i += 256) {
    const int tt = i & 15, d = i >> 4;
    const int32_t sl = slot_s[tt];
    if (sl < 0) continue;
    const int32_t blk = sl / BS, off = sl % BS;
    v_cache[((static_cast<int64_t>(blk) * H_kv + h) * D + d) * BS + off] =
        encode<NewT, CacheT>(v_s[tt][d], v_inv);
  }
}

// grid: (ceil(n / 16), H_kv); block: 256 threads.
template <typename NewT, typename CacheT, int D, int BS>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const typename NewT::raw* __restrict__ k_new, const typename NewT::raw* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t n, typename CacheT::raw* __restrict__ k_cache,
    typename CacheT::raw* __restrict__ v_cache, int32_t num_blocks, int32_t H_kv, float k_inv,
    float v_inv) {
  cw_tile<NewT, CacheT, D, false, BS>(blockIdx.x, blockIdx.y, k_new, v_new, slots, n, k_cache,
                                      v_cache, num_blocks, H_kv, k_inv, v_inv);
}

// grid: stage groups + ceil(n / 16) * H_kv; block: 256 threads.  The first
// `sgroups` work-groups copy the metadata buffer (as pa_stage), the others
// scatter the new tokens with the slot mapping read from the same pinned
// buffer, so both run in one launch.  With `tables`, the work-groups of KV
// head 0 also enter each token's block in row i of the device block tables
// at the column of its position (context length - 1, read from the pinned
// buffer as well).
template <typename NewT, typename CacheT, int D, typename W>
__global__ __launch_bounds__(256) void stage_cache_write_kernel(
    W* __restrict__ dst, const W* __restrict__ src, int64_t n_words, int32_t sgroups,
    const typename NewT::raw* __restrict__ k_new, const typename NewT::raw* __restrict__ v_new,
    const int32_t* __restrict__ slots_host, int32_t n, typename CacheT::raw* __restrict__ k_cache,
    typename CacheT::raw* __restrict__ v_cache, int32_t num_blocks, int32_t H_kv, float k_inv,
    float v_inv, int32_t* __restrict__ tables, int32_t max_blocks,
    const int32_t* __restrict__ lens_host) {
  const int b = blockIdx.x;
  if (b < sgroups) {
    stage_words<W>(dst, src, n_words, b, sgroups);
    return;
  }
  const int ntb = (n + 15) / 16;
  const int r = b - sgroups;
  if (tables && r < ntb && threadIdx.x < 16) {
    const int64_t t = static_cast<int64_t>(r) * 16 + threadIdx.x;
    if (t < n) {
      const int32_t sl = __hip_atomic_load(slots_host + t, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
      const int32_t len = __hip_atomic_load(lens_host + t, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
      if (sl >= 0 && sl < num_blocks * kBlock && len >= 1 &&
          len <= static_cast<int64_t>(max_blocks) * kBlock)
        tables[t * max_blocks + (len - 1) / kBlock] = sl / kBlock;
    }
  }
  cw_tile<NewT, CacheT, D, true, kBlock>(r % ntb, r / ntb, k_new, v_new, slots_host, n, k_cache,
                                         v_cache, num_blocks, H_kv, k_inv, v_inv);
}

template <typename NewT, typename CacheT, int D, int BS>
static pa_status launch_cw(hipStream_t st, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                           int32_t num_blocks, int32_t H_kv, float k_inv, float v_inv) {
  dim3 grid((n + 15) / 16, H_kv);
  hipError_t e = launch(kCacheWrite, cache_write_kernel<NewT, CacheT, D, BS>, grid, dim3(256), 0, st,
                        static_cast<const typename NewT::raw*>(k_new),
                        static_cast<const typename NewT::raw*>(v_new), slots, n,
                        static_cast<typename CacheT::raw*>(k_cache),
                        static_cast<typename CacheT::raw*>(v_cache), num_blocks, H_kv, k_inv,
                        v_inv);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_cache_write: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

template <typename NewT, typename CacheT, int BS>
static pa_status launch_cw_d(hipStream_t st, const void* k_new, const void* v_new,
                             const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                             int32_t num_blocks, int32_t H_kv, int32_t D, float k_inv,
                             float v_inv) {
  if (D == 128)
    return launch_cw<NewT, CacheT, 128, BS>(st, k_new, v_new, slots, n, k_cache, v_cache,
                                            num_blocks, H_kv, k_inv, v_inv);
  return launch_cw<NewT, CacheT, 64, BS>(st, k_new, v_new, slots, n, k_cache, v_cache, num_blocks,
                                         H_kv, k_inv, v_inv);
}

template <typename NewT, typename CacheT>
static pa_status launch_cache_write(hipStream_t st, const void* k_new, const void* v_new,
                                    const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                                    float k_inv, float v_inv) {
  if (bs == 8)
    return launch_cw_d<NewT, CacheT, 8>(st, k_new, v_new, slots, n, k_cache, v_cache, num_blocks,
                                        H_kv, D, k_inv, v_inv);
  if (bs == 32)
    return launch_cw_d<NewT, CacheT, 32>(st, k_new, v_new, slots, n, k_cache, v_cache,
                                         num_blocks, H_kv, D, k_inv, v_inv);
  return launch_cw_d<NewT, CacheT, 16>(st, k_new, v_new, slots, n, k_cache, v_cache, num_blocks,
                                       H_kv, D, k_inv, v_inv);
}

// Argument checks shared by pa_cache_write and pa_stage_cache_write (all but
// the slot mapping); on success `combo` names the (new, cache) types: 0 f32
// into f32, 1 bf16 into bf16, 2 bf16 into fp8, with the reciprocal scales.
struct CwPlan {
  int combo = 0;
  float k_inv = 1.f, v_inv = 1.f;
};

static pa_status cw_check(const char* who, const void* k_new, const void* v_new, pa_dtype new_dt,
                          int32_t n, void* k_cache, void* v_cache, pa_dtype cache_dt,
                          int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs, float k_scale,
                          float v_scale, CwPlan* plan, bool any_bs = false) {
  if (any_bs ? (bs != 8 && bs != 16 && bs != 32) : bs != kBlock)
    return fail(PA_ERR_INVALID, "%s: block size %d not in %s", who, bs,
                any_bs ? "{8, 16, 32}" : "{16}");
  if (n < 0 || H_kv <= 0 || num_blocks < 0)
    return fail(PA_ERR_INVALID, "%s: n=%d H_kv=%d num_blocks=%d", who, n, H_kv, num_blocks);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "%s: D=%d not in {64,128}", who, D);
  if (static_cast<int64_t>(num_blocks) * bs > INT32_MAX)
    return fail(PA_ERR_INVALID, "%s: num_blocks=%d overflows int32 slots", who, num_blocks);
  if (H_kv > 65535) return fail(PA_ERR_INVALID, "%s: H_kv=%d too large", who, H_kv);
  if (n > 0 && (!k_new || !v_new || !k_cache || !v_cache))
    return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  if (new_dt == PA_F32 && cache_dt == PA_F32) {
    plan->combo = 0;
  } else if (new_dt == PA_BF16 && cache_dt == PA_BF16) {
    plan->combo = 1;
  } else if (new_dt == PA_BF16 && cache_dt == PA_FP8_E4M3) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
        !__builtin_isfinite(v_scale))
      return fail(PA_ERR_INVALID, "%s: fp8 scales must be finite and > 0", who);
    plan->combo = 2;
    // one fp32 reciprocal each, computed here once
    plan->k_inv = 1.0f / k_scale;
    plan->v_inv = 1.0f / v_scale;
  } else {
    return fail(PA_ERR_INVALID, "%s: unsupported dtypes new=%d cache=%d", who, new_dt, cache_dt);
  }
  return PA_OK;
}

// Block-table upkeep of a decode batch (pa_stage_decode_append); none for
// pa_stage_cache_write.
struct TableUpkeep {
  int32_t* tables = nullptr;
  int32_t max_blocks = 0;
  const int32_t* lens_dev = nullptr;
};

template <typename NewT, typename CacheT, int D, typename W>
static pa_status launch_scw(hipStream_t st, void* dst, const void* src_dev, size_t bytes,
                            const int32_t* slots_dev, const void* k_new, const void* v_new,
                            int32_t n, void* k_cache, void* v_cache, int32_t num_blocks,
                            int32_t H_kv, float k_inv, float v_inv, const TableUpkeep& tu) {
  const int64_t n_words = static_cast<int64_t>(bytes / sizeof(W));
  const int sgroups = stage_groups(n_words);
  const int64_t grid = sgroups + static_cast<int64_t>((n + 15) / 16) * H_kv;
  if (grid > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_stage_cache_write: grid too large (%lld)",
                static_cast<long long>(grid));
  hipError_t e = launch(kStageCacheWrite, stage_cache_write_kernel<NewT, CacheT, D, W>,
                        dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, static_cast<W*>(dst),
                        static_cast<const W*>(src_dev), n_words, sgroups,
                        static_cast<const typename NewT::raw*>(k_new),
                        static_cast<const typename NewT::raw*>(v_new), slots_dev, n,
                        static_cast<typename CacheT::raw*>(k_cache),
                        static_cast<typename CacheT::raw*>(v_cache), num_blocks, H_kv, k_inv,
                        v_inv, tu.tables, tu.max_blocks, tu.lens_dev);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_stage_cache_write: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

template <typename NewT, typename CacheT, typename W>
static pa_status launch_scw_d(int32_t D, hipStream_t st, void* dst, const void* src_dev,
                              size_t bytes, const int32_t* slots_dev, const void* k_new,
                              const void* v_new, int32_t n, void* k_cache, void* v_cache,
                              int32_t num_blocks, int32_t H_kv, float k_inv, float v_inv,
                              const TableUpkeep& tu) {
  if (D == 128)
    return launch_scw<NewT, CacheT, 128, W>(st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                            k_cache, v_cache, num_blocks, H_kv, k_inv, v_inv, tu);
  return launch_scw<NewT, CacheT, 64, W>(st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                         k_cache, v_cache, num_blocks, H_kv, k_inv, v_inv, tu);
}

template <typename W>
static pa_status launch_scw_types(const CwPlan& plan, int32_t D, hipStream_t st, void* dst,
                                  const void* src_dev, size_t bytes, const int32_t* slots_dev,
                                  const void* k_new, const void* v_new, int32_t n, void* k_cache,
                                  void* v_cache, int32_t num_blocks, int32_t H_kv,
                                  const TableUpkeep& tu) {
  if (plan.combo == 0)
    return launch_scw_d<F32, F32, W>(D, st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                     k_cache, v_cache, num_blocks, H_kv, 1.f, 1.f, tu);
  if (plan.combo == 1)
    return launch_scw_d<BF16, BF16, W>(D, st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                       k_cache, v_cache, num_blocks, H_kv, 1.f, 1.f, tu);
  return launch_scw_d<BF16, FP8, W>(D, st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                    k_cache, v_cache, num_blocks, H_kv, plan.k_inv, plan.v_inv,
                                    tu);
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_cache_write(void* stream, const void* k_new, const void* v_new,
                                    pa_dtype new_dt, const int32_t* slot_mapping, int32_t n,
                                    void* k_cache, void* v_cache, pa_dtype cache_dt,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                                    float k_scale, float v_scale) {
  CwPlan plan;
  const pa_status chk = cw_check("pa_cache_write", k_new, v_new, new_dt, n, k_cache, v_cache,
                                 cache_dt, num_blocks, H_kv, D, bs, k_scale, v_scale, &plan, true);
  if (chk != PA_OK) return chk;
  if (n == 0) return PA_OK;
  if (!slot_mapping) return fail(PA_ERR_INVALID, "pa_cache_write: NULL buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.combo == 0)
    return launch_cache_write<F32, F32>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                        num_blocks, H_kv, D, bs, 1.f, 1.f);
  if (plan.combo == 1)
    return launch_cache_write<BF16, BF16>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                          num_blocks, H_kv, D, bs, 1.f, 1.f);
  return launch_cache_write<BF16, FP8>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                       num_blocks, H_kv, D, bs, plan.k_inv, plan.v_inv);
}

namespace pa {

static pa_status stage_cache_write_impl(const char* who, void* stream, void* dst,
                                        const void* src_host, size_t bytes, size_t slot_offset,
                                        const void* k_new, const void* v_new, pa_dtype new_dt,
                                        int32_t n, void* k_cache, void* v_cache,
                                        pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv,
                                        int32_t D, int32_t bs, float k_scale, float v_scale,
                                        const size_t* lens_offset, int32_t* block_tables,
                                        int32_t max_blocks) {
  CwPlan plan;
  const pa_status chk = cw_check(who, k_new, v_new, new_dt, n, k_cache, v_cache, cache_dt,
                                 num_blocks, H_kv, D, bs, k_scale, v_scale, &plan);
  if (chk != PA_OK) return chk;
  if (bytes % 4 != 0 || slot_offset % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(src_host) % 4 != 0)
    return fail(PA_ERR_INVALID,
                "%s: bytes=%zu, slot_offset=%zu and both addresses must be multiples of 4", who,
                bytes, slot_offset);
  if (n > 0 && (slot_offset > bytes || (bytes - slot_offset) / 4 < static_cast<size_t>(n)))
    return fail(PA_ERR_INVALID, "%s: %d slots at byte %zu do not fit the %zu-byte buffer", who, n,
                slot_offset, bytes);
  if (lens_offset) {
    if (*lens_offset % 4 != 0)
      return fail(PA_ERR_INVALID, "%s: lens_offset=%zu must be a multiple of 4", who,
                  *lens_offset);
    if (n > 0 && (*lens_offset > bytes || (bytes - *lens_offset) / 4 < static_cast<size_t>(n)))
      return fail(PA_ERR_INVALID, "%s: %d lengths at byte %zu do not fit the %zu-byte buffer",
                  who, n, *lens_offset, bytes);
    if (max_blocks < 1) return fail(PA_ERR_INVALID, "%s: max_blocks=%d < 1", who, max_blocks);
    if (n > 0 && !block_tables) return fail(PA_ERR_INVALID, "%s: NULL block_tables", who);
  }
  if (bytes == 0) return PA_OK;  // and n == 0
  if (!dst || !src_host) return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  void* src_dev = nullptr;
  const pa_status ps = pinned_alias(who, src_host, &src_dev);
  if (ps != PA_OK) return ps;
  const int32_t* slots_dev =
      reinterpret_cast<const int32_t*>(static_cast<const char*>(src_dev) + slot_offset);
  TableUpkeep tu;
  if (lens_offset && n > 0) {
    tu.tables = block_tables;
    tu.max_blocks = max_blocks;
    tu.lens_dev =
        reinterpret_cast<const int32_t*>(static_cast<const char*>(src_dev) + *lens_offset);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (bytes % 8 == 0 && reinterpret_cast<uintptr_t>(dst) % 8 == 0 &&
      reinterpret_cast<uintptr_t>(src_dev) % 8 == 0)
    return launch_scw_types<uint64_t>(plan, D, st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                      k_cache, v_cache, num_blocks, H_kv, tu);
  return launch_scw_types<uint32_t>(plan, D, st, dst, src_dev, bytes, slots_dev, k_new, v_new, n,
                                    k_cache, v_cache, num_blocks, H_kv, tu);
}

}  // namespace pa

extern "C" pa_status pa_stage_cache_write(void* stream, void* dst, const void* src_host,
                                          size_t bytes, size_t slot_offset, const void* k_new,
                                          const void* v_new, pa_dtype new_dt, int32_t n,
                                          void* k_cache, void* v_cache, pa_dtype cache_dt,
                                          int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                                          float k_scale, float v_scale) {
  return stage_cache_write_impl("pa_stage_cache_write", stream, dst, src_host, bytes,
                                slot_offset, k_new, v_new, new_dt, n, k_cache, v_cache, cache_dt,
                                num_blocks, H_kv, D, bs, k_scale, v_scale, nullptr, nullptr, 0);
}

extern "C" pa_status pa_stage_decode_append(void* stream, void* dst, const void* src_host,
                                            size_t bytes, size_t slot_offset, size_t lens_offset,
                                            const void* k_new, const void* v_new, pa_dtype new_dt,
                                            int32_t n, void* k_cache, void* v_cache,
                                            pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv,
                                            int32_t D, int32_t bs, float k_scale, float v_scale,
                                            int32_t* block_tables, int32_t max_blocks) {
  return stage_cache_write_impl("pa_stage_decode_append", stream, dst, src_host, bytes,
                                slot_offset, k_new, v_new, new_dt, n, k_cache, v_cache, cache_dt,
                                num_blocks, H_kv, D, bs, k_scale, v_scale, &lens_offset,
                                block_tables, max_blocks);
}

extern "C" pa_status pa_decode_append(void* stream, const int32_t* slots, const int32_t* lens,
                                      int32_t n, const void* k_new, const void* v_new,
                                      pa_dtype new_dt, void* k_cache, void* v_cache,
                                      pa_dtype cache_dt, int32_t num_blocks, int32_t H_kv,
                                      int32_t D, int32_t bs, float k_scale, float v_scale,
                                      int32_t* block_tables, int32_t max_blocks) {
  const char* who = "pa_decode_append";
  CwPlan plan;
  const pa_status chk = cw_check(who, k_new, v_new, new_dt, n, k_cache, v_cache, cache_dt,
                                 num_blocks, H_kv, D, bs, k_scale, v_scale, &plan);
  if (chk != PA_OK) return chk;
  if (max_blocks < 1) return fail(PA_ERR_INVALID, "%s: max_blocks=%d < 1", who, max_blocks);
  if (n == 0) return PA_OK;
  if (!slots || !lens || !block_tables) return fail(PA_ERR_INVALID, "%s: NULL buffer", who);
  TableUpkeep tu;
  tu.tables = block_tables;
  tu.max_blocks = max_blocks;
  tu.lens_dev = lens;
  // no words to stage: every work-group writes K/V (and table entries)
  return launch_scw_types<uint64_t>(plan, D, static_cast<hipStream_t>(stream), nullptr, nullptr, 0,
                                    slots, k_new, v_new, n, k_cache, v_cache, num_blocks, H_kv,
                                    tu);
}
