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

// grid: (ceil(n / 16), H_kv); block: 256 threads.
template <typename NewT, typename CacheT, int D>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const typename NewT::raw* __restrict__ k_new, const typename NewT::raw* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t n, typename CacheT::raw* __restrict__ k_cache,
    typename CacheT::raw* __restrict__ v_cache, int32_t num_blocks, int32_t H_kv, float k_inv,
    float v_inv) {
  using NR = typename NewT::raw;
  using CR = typename CacheT::raw;
  constexpr int X = 16 / sizeof(CR);  // cache elements per 16-byte chunk
  constexpr int NCH = D / X;          // chunks per token row
  __shared__ NR v_s[16][D + 2];
  __shared__ int32_t slot_s[16];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
  if (tid < 16) {
    const int64_t t = t0 + tid;
    int32_t sl = t < n ? slots[t] : -1;
    if (sl >= num_blocks * kBlock) sl = -1;
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
    const int32_t blk = sl / kBlock, off = sl % kBlock;
    const NR* src = k_new + (t * H_kv + h) * D + ch * X;
    CR* dst = k_cache + ((static_cast<int64_t>(blk) * H_kv + h) * NCH + ch) * (kBlock * X) + off * X;
#pragma unroll
    for (int j = 0; j < X; ++j) dst[j] = encode<NewT, CacheT>(src[j], k_inv);
  }
  // V: thread -> (d, token), 16 adjacent threads share d
  for (int i = tid; i < 16 * D; i += 256) {
    const int tt = i & 15, d = i >> 4;
    const int32_t sl = slot_s[tt];
    if (sl < 0) continue;
    const int32_t blk = sl / kBlock, off = sl % kBlock;
    v_cache[((static_cast<int64_t>(blk) * H_kv + h) * D + d) * kBlock + off] =
        encode<NewT, CacheT>(v_s[tt][d], v_inv);
  }
}

template <typename NewT, typename CacheT, int D>
static pa_status launch_cw(hipStream_t st, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                           int32_t num_blocks, int32_t H_kv, float k_inv, float v_inv) {
  dim3 grid((n + 15) / 16, H_kv);
  hipError_t e = launch(kCacheWrite, cache_write_kernel<NewT, CacheT, D>, grid, dim3(256), 0, st,
                        static_cast<const typename NewT::raw*>(k_new),
                        static_cast<const typename NewT::raw*>(v_new), slots, n,
                        static_cast<typename CacheT::raw*>(k_cache),
                        static_cast<typename CacheT::raw*>(v_cache), num_blocks, H_kv, k_inv,
                        v_inv);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_cache_write: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

template <typename NewT, typename CacheT>
static pa_status launch_cache_write(hipStream_t st, const void* k_new, const void* v_new,
                                    const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, float k_inv,
                                    float v_inv) {
  if (D == 128)
    return launch_cw<NewT, CacheT, 128>(st, k_new, v_new, slots, n, k_cache, v_cache, num_blocks,
                                        H_kv, k_inv, v_inv);
  return launch_cw<NewT, CacheT, 64>(st, k_new, v_new, slots, n, k_cache, v_cache, num_blocks,
                                     H_kv, k_inv, v_inv);
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_cache_write(void* stream, const void* k_new, const void* v_new,
                                    pa_dtype new_dt, const int32_t* slot_mapping, int32_t n,
                                    void* k_cache, void* v_cache, pa_dtype cache_dt,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                                    float k_scale, float v_scale) {
  if (bs != kBlock) return fail(PA_ERR_INVALID, "pa_cache_write: block size %d != 16", bs);
  if (n < 0 || H_kv <= 0 || num_blocks < 0)
    return fail(PA_ERR_INVALID, "pa_cache_write: n=%d H_kv=%d num_blocks=%d", n, H_kv,
                num_blocks);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "pa_cache_write: D=%d not in {64,128}", D);
  if (static_cast<int64_t>(num_blocks) * kBlock > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_cache_write: num_blocks=%d overflows int32 slots", num_blocks);
  if (H_kv > 65535) return fail(PA_ERR_INVALID, "pa_cache_write: H_kv=%d too large", H_kv);
  if (n == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID, "pa_cache_write: NULL buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (new_dt == PA_F32 && cache_dt == PA_F32)
    return launch_cache_write<F32, F32>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                        num_blocks, H_kv, D, 1.f, 1.f);
  if (new_dt == PA_BF16 && cache_dt == PA_BF16)
    return launch_cache_write<BF16, BF16>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                          num_blocks, H_kv, D, 1.f, 1.f);
  if (new_dt == PA_BF16 && cache_dt == PA_FP8_E4M3) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
        !__builtin_isfinite(v_scale))
      return fail(PA_ERR_INVALID, "pa_cache_write: fp8 scales must be finite and > 0");
    // one fp32 reciprocal each, computed here once
    const float k_inv = 1.0f / k_scale;
    const float v_inv = 1.0f / v_scale;
    return launch_cache_write<BF16, FP8>(st, k_new, v_new, slot_mapping, n, k_cache, v_cache,
                                         num_blocks, H_kv, D, k_inv, v_inv);
  }
  return fail(PA_ERR_INVALID, "pa_cache_write: unsupported dtypes new=%d cache=%d", new_dt,
              cache_dt);
}
