// pa_cache_write: scatter new K/V vectors into the paged cache.
//
// LESSON "vLLM Serving Internals", "The Concept: PagedAttention as a virtual
// memory system": the K/V of token position p of a sequence live in block
// table[p / bs] at offset p % bs.  The host turns positions into flat slots
// (block * bs + offset); this kernel stores each token's K row and V column
// at its slot for every KV head, optionally quantising bf16 to fp8 e4m3fn
// with a per-tensor scale.
//
// Layout: K cache [nb][H_kv][16][D] (row per token), V cache [nb][H_kv][D][16]
// (column per token).  One work-group handles 16 consecutive tokens of the
// input and one KV head; when those tokens fill one block in order (the
// prefill case) every V row of 16 tokens is written by 16 adjacent lanes.
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
// Thread (tt, dd) with tt = tid % 16 (token of the group), dd = tid / 16
// walks d = dd, dd + 16, ... so that, for the V column writes, 16 adjacent
// lanes cover one 16-token row of a block.
template <typename NewT, typename CacheT>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const typename NewT::raw* __restrict__ k_new, const typename NewT::raw* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t n, typename CacheT::raw* __restrict__ k_cache,
    typename CacheT::raw* __restrict__ v_cache, int32_t num_blocks, int32_t H_kv, int32_t D,
    float k_inv, float v_inv) {
  const int tt = threadIdx.x & 15;
  const int dd = threadIdx.x >> 4;
  const int h = blockIdx.y;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + tt;
  if (t >= n) return;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * kBlock) return;
  const int32_t blk = slot / kBlock;
  const int32_t off = slot % kBlock;
  const int64_t src = (t * H_kv + h) * D;
  const int64_t tile = (static_cast<int64_t>(blk) * H_kv + h) * kBlock * D;
  for (int d = dd; d < D; d += 16) {
    k_cache[tile + static_cast<int64_t>(off) * D + d] = encode<NewT, CacheT>(k_new[src + d], k_inv);
    v_cache[tile + static_cast<int64_t>(d) * kBlock + off] =
        encode<NewT, CacheT>(v_new[src + d], v_inv);
  }
}

template <typename NewT, typename CacheT>
static pa_status launch_cache_write(hipStream_t st, const void* k_new, const void* v_new,
                                    const int32_t* slots, int32_t n, void* k_cache, void* v_cache,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, float k_inv,
                                    float v_inv) {
  dim3 grid((n + 15) / 16, H_kv);
  hipLaunchKernelGGL((cache_write_kernel<NewT, CacheT>), grid, dim3(256), 0, st,
                     static_cast<const typename NewT::raw*>(k_new),
                     static_cast<const typename NewT::raw*>(v_new), slots, n,
                     static_cast<typename CacheT::raw*>(k_cache),
                     static_cast<typename CacheT::raw*>(v_cache), num_blocks, H_kv, D, k_inv,
                     v_inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_cache_write: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_cache_write(void* stream, const void* k_new, const void* v_new,
                                    pa_dtype new_dt, const int32_t* slot_mapping, int32_t n,
                                    void* k_cache, void* v_cache, pa_dtype cache_dt,
                                    int32_t num_blocks, int32_t H_kv, int32_t D, int32_t bs,
                                    float k_scale, float v_scale) {
  if (bs != kBlock) return fail(PA_ERR_INVALID, "pa_cache_write: block size %d != 16", bs);
  if (n < 0 || H_kv <= 0 || D <= 0 || num_blocks < 0)
    return fail(PA_ERR_INVALID, "pa_cache_write: n=%d H_kv=%d D=%d num_blocks=%d", n, H_kv, D,
                num_blocks);
  if (static_cast<int64_t>(num_blocks) * kBlock > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_cache_write: num_blocks=%d overflows int32 slots", num_blocks);
  if (n == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID, "pa_cache_write: NULL buffer");
  if (H_kv > 65535) return fail(PA_ERR_INVALID, "pa_cache_write: H_kv=%d too large", H_kv);
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
