// pa_decode: one query token per sequence attends its paged K/V.
//
// ARTICLE "vLLM inference engine architecture" (lpnh.cn) §2.3: the kernel
// finds a query's K/V blocks through block_tables up to context_lens,
// computes scores within a block and accumulates across blocks.  Here the
// accumulation is an online softmax (running max m, running sum l,
// unnormalised output o) and the blocks of a long context are cut into
// fixed-length splits processed by different waves; a second kernel merges
// the split partials exactly:
//     m* = max_j m_j,  l* = sum_j l_j 2^(m_j - m*),
//     out = sum_j o_j 2^(m_j - m*) / l*.
// (Scores are kept in base 2: s = sm_scale * log2(e) * q.k, so exp becomes
// the hardware exp2.)
//
// Grouped-query heads (query head h reads KV head h / G, G = H_q / H_kv) share
// every K/V byte: one wave computes all G heads of its KV head, so each
// K/V tile is read from HBM once per KV head.
//
// Matrix-core mapping (gfx950 v_mfma_f32_16x16x32_bf16, wave64):
//   scores  S^T[token][head] = K[token][:] . Q^T[:][head]
//           A = K tile (16 tokens x 32 dims per step), B = Q^T (32 dims x 16
//           head columns, heads >= G zero-padded)
//   output  O^T[d][head] += V^T[d][token] . P^T[token][head]
//           A = V^T (16 dims x 32 tokens) read straight from the token-minor
//           V tile, B = P^T taken from the score registers without any
//           lane exchange.
// Two 16-token blocks (32 tokens) form one step.  Lane l (c = l % 16,
// g = l / 16) holds, after the score products, the scores of 8 consecutive
// positions of head column c: block (g < 2 ? first : second), tokens
// 8 * (g % 2) + 0..7.  The K rows are assigned to MFMA rows so that this
// holds: score tile X row 4a + r is token 8 * (a % 2) + r of block a / 2,
// tile Y row 4a + r is that token + 4.
//
// Every lane loads 16 contiguous bytes per operand (bf16) straight from HBM
// into the operand registers; the next step's tiles are loaded while the
// current step computes.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kDecodeWaves = 4;       // waves per work-group, one split each
constexpr int kSplitTokens = 256;     // tokens per split (a multiple of 32)
constexpr int kSplitBlocks = kSplitTokens / kBlock;

inline int32_t decode_num_splits(int32_t max_context_len) {
  const int32_t nblk = (max_context_len + kBlock - 1) / kBlock;
  return nblk <= 0 ? 1 : (nblk + kSplitBlocks - 1) / kSplitBlocks;
}

// Dimension index of k-slot group (step s, lane group g) in a D-vector: the
// 8 consecutive dims a lane feeds to one MFMA.  bf16 rows: each step covers a
// 64-byte run per token row (4 lane groups side by side); fp8 rows: a lane's
// D/32 steps cover one run of D/4 bytes.
template <typename CacheT, int D>
__device__ __forceinline__ int kdim(int s, int g) {
  if constexpr (sizeof(typename CacheT::raw) == 1)
    return (D / 4) * g + 8 * s;
  else
    return 32 * s + 8 * g;
}

template <typename CacheT, int D>
struct StepRegs;

template <int D>
struct StepRegs<BF16, D> {
  bf16x8 kx[D / 32], ky[D / 32], v[D / 16];
};

template <int D>
struct StepRegs<FP8, D> {
  u32x4 kx[D / 64], ky[D / 64];  // D/4 fp8 codes per lane per tile
  u32x2 v[D / 16];
};

template <typename CacheT, int D>
__device__ __forceinline__ void load_step(StepRegs<CacheT, D>& r,
                                          const typename CacheT::raw* __restrict__ k_cache,
                                          const typename CacheT::raw* __restrict__ v_cache,
                                          int64_t tile_a, int64_t tile_b, int c, int g) {
  // K rows: tile X row c -> token 8*((c>>2)&1) + (c&3) of block (c>>3 ? b : a)
  const int krow_blk = c >> 3;
  const int ktok = 8 * ((c >> 2) & 1) + (c & 3);
  const int64_t ktile = krow_blk ? tile_b : tile_a;
  const typename CacheT::raw* kx = k_cache + ktile * (kBlock * D) + ktok * D;
  const typename CacheT::raw* ky = kx + 4 * D;
  // V: lane group g reads block (g >> 1), tokens 8*(g&1) .. +8 of row d
  const int64_t vtile = (g >> 1) ? tile_b : tile_a;
  const typename CacheT::raw* vp = v_cache + vtile * (kBlock * D) + c * kBlock + 8 * (g & 1);
  if constexpr (sizeof(typename CacheT::raw) == 2) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      r.kx[s] = *reinterpret_cast<const bf16x8*>(kx + kdim<CacheT, D>(s, g));
      r.ky[s] = *reinterpret_cast<const bf16x8*>(ky + kdim<CacheT, D>(s, g));
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      r.v[t] = *reinterpret_cast<const bf16x8*>(vp + 16 * t * kBlock);
  } else {
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      r.kx[s] = *reinterpret_cast<const u32x4*>(kx + (D / 4) * g + 16 * s);
      r.ky[s] = *reinterpret_cast<const u32x4*>(ky + (D / 4) * g + 16 * s);
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      r.v[t] = *reinterpret_cast<const u32x2*>(vp + 16 * t * kBlock);
  }
}

template <typename CacheT, int D>
__device__ __forceinline__ bf16x8 k_operand(const StepRegs<CacheT, D>& r, bool y, int s) {
  if constexpr (sizeof(typename CacheT::raw) == 2) {
    return y ? r.ky[s] : r.kx[s];
  } else {
    // fp8: kdim = (D/4)*g + 8*s -> step s is dwords (2s, 2s+1) of the lane's run
    const u32x4 w = y ? r.ky[s >> 1] : r.kx[s >> 1];
    u32x2 pair;
    pair[0] = (s & 1) ? w[2] : w[0];
    pair[1] = (s & 1) ? w[3] : w[1];
    return fp8x8_to_bf16x8(pair);
  }
}

template <typename CacheT, int D>
__device__ __forceinline__ bf16x8 v_operand(const StepRegs<CacheT, D>& r, int t) {
  if constexpr (sizeof(typename CacheT::raw) == 2)
    return r.v[t];
  else
    return fp8x8_to_bf16x8(r.v[t]);
}

// Workspace of the matrix-core path: completion counters (one int32 per
// (sequence, KV head), zero between calls), then per (sequence, query head,
// split) the running max and sum (2 floats) and the unnormalised output
// (D floats).
inline size_t decode_counter_bytes(int32_t S, int32_t H_kv) {
  return (static_cast<size_t>(S) * H_kv * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

template <typename OutT>
__device__ __forceinline__ void store_out4(typename OutT::raw* dst, f32x4 v) {
  if constexpr (sizeof(typename OutT::raw) == 2) {
    u32x2 w;
    w[0] = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    w[1] = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<u32x2*>(dst) = w;
  } else {
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// grid: (ceil(n_splits / kDecodeWaves), H_kv, S); block: 64 * kDecodeWaves.
// Wave w of work-group x handles split x * kDecodeWaves + w of (seq, kv head).
// A context that fits one split is finished by its wave directly.  Otherwise
// each wave stores its partial (m, l, o) and bumps the (seq, kv head)
// counter; the wave that arrives last merges all partials and writes the
// output, then clears the counter for the next call.
template <typename CacheT, int D>
__global__ __launch_bounds__(kWave* kDecodeWaves) void decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, int32_t num_blocks, const int32_t* __restrict__ context_lens,
    int32_t H_q, int32_t H_kv, int32_t G, int32_t n_splits, float score_scale, float out_scale,
    int32_t* __restrict__ counters, float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int split = blockIdx.x * kDecodeWaves + wave;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  if (split >= n_splits) return;

  const int32_t L = min(context_lens[seq], max_blocks * kBlock);
  const int32_t nblk = (L + kBlock - 1) / kBlock;
  const int32_t b0 = split * kSplitBlocks;
  if (L <= 0 || b0 >= nblk) return;
  const int32_t n_valid = min(n_splits, (nblk + kSplitBlocks - 1) / kSplitBlocks);
  const int32_t b1 = (split == n_splits - 1) ? nblk : min(nblk, b0 + kSplitBlocks);
  const int32_t* __restrict__ table = block_tables + static_cast<int64_t>(seq) * max_blocks;

  // Q^T operand: column c = head kvh*G + c, zero for padded columns.
  bf16x8 qb[D / 32];
  {
    const bool live = c < G;
    const uint16_t* qp = q + (static_cast<int64_t>(seq) * H_q + kvh * G + (live ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + kdim<CacheT, D>(s, g));
      qb[s] = live ? v : bf16x8{};
    }
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  auto tile_of = [&](int32_t b) -> int64_t {
    return static_cast<int64_t>(safe_block(table[b], num_blocks)) * H_kv + kvh;
  };

  StepRegs<CacheT, D> cur, nxt;
  int32_t p = b0;
  {
    const int64_t ta = tile_of(p);
    const int64_t tb = (p + 1 < b1) ? tile_of(p + 1) : ta;
    load_step<CacheT, D>(cur, k_cache, v_cache, ta, tb, c, g);
  }
  for (; p < b1; p += 2) {
    const int32_t pn = p + 2;
    if (pn < b1) {
      const int64_t ta = tile_of(pn);
      const int64_t tb = (pn + 1 < b1) ? tile_of(pn + 1) : ta;
      load_step<CacheT, D>(nxt, k_cache, v_cache, ta, tb, c, g);
    }
    // scores of the 32 tokens of this step
    f32x4 sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      sx = mfma16x16x32(k_operand(cur, false, s), qb[s], sx);
      sy = mfma16x16x32(k_operand(cur, true, s), qb[s], sy);
    }
    const int32_t pos0 = (p + (g >> 1)) * kBlock + 8 * (g & 1);
    float sc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = (pos0 + j < L) ? sx[j] * score_scale : -__builtin_inff();
      sc[j + 4] = (pos0 + 4 + j < L) ? sy[j] * score_scale : -__builtin_inff();
    }
    float mx = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = __builtin_amdgcn_exp2f(sc[j] - m_new);
      psum += e;
      pb[j] = static_cast<__bf16>(e);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      o[t] *= alpha;
      o[t] = mfma16x16x32(v_operand(cur, t), pb, o[t]);
    }
    cur = nxt;
  }
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  const int64_t head_row = static_cast<int64_t>(seq) * H_q + kvh * G + c;  // valid if c < G
  if (n_valid == 1) {
    if (c < G) {
      const float inv = out_scale / l_run;
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        store_out4<BF16>(out + head_row * D + 16 * t + 4 * g, o[t] * inv);
    }
    return;
  }

  const int64_t part = head_row * n_splits + split;
  if (c < G) {
    float* dst = ws_o + part * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * g) = o[t];
    if (g == 0) {
      ws_ml[part * 2 + 0] = m_run;
      ws_ml[part * 2 + 1] = l_run;
    }
  }
  // publish the partial, then count this split as done
  __threadfence();
  int32_t* ctr = counters + static_cast<int64_t>(seq) * H_kv + kvh;
  int32_t prev = 0;
  if (lane == 0) prev = atomicAdd(ctr, 1);
  prev = __shfl(prev, 0, kWave);
  if (prev != n_valid - 1) return;
  // last arrival: every other split's partial is visible after this fence
  __threadfence();
  if (lane == 0) atomicExch(ctr, 0);
  if (c >= G) return;
  const int64_t base = head_row * n_splits;
  float M = -__builtin_inff();
  for (int j = 0; j < n_valid; ++j) M = fmaxf(M, ws_ml[(base + j) * 2]);
  float tot = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n_valid; ++j) {
    const float w = __builtin_amdgcn_exp2f(ws_ml[(base + j) * 2] - M);
    tot += w * ws_ml[(base + j) * 2 + 1];
    const float* src = ws_o + (base + j) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      acc[t] += w * *reinterpret_cast<const f32x4*>(src + 16 * t + 4 * g);
  }
  const float inv = out_scale / tot;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) store_out4<BF16>(out + head_row * D + 16 * t + 4 * g, acc[t] * inv);
}

template <typename CacheT, int D>
static pa_status launch_decode_mfma(hipStream_t st, void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    int32_t max_blocks, int32_t num_blocks,
                                    const int32_t* context_lens, int32_t S, int32_t H_q,
                                    int32_t H_kv, int32_t max_context_len, float sm_scale,
                                    float k_scale, float v_scale, void* ws) {
  const int32_t n_splits = decode_num_splits(max_context_len);
  int32_t* counters = static_cast<int32_t*>(ws);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + decode_counter_bytes(S, H_kv));
  float* ws_o = ws_ml + static_cast<int64_t>(S) * H_q * n_splits * 2;
  const float score_scale = sm_scale * kLog2e * k_scale;
  dim3 grid((n_splits + kDecodeWaves - 1) / kDecodeWaves, H_kv, S);
  hipLaunchKernelGGL((decode_kernel<CacheT, D>), grid, dim3(kWave * kDecodeWaves), 0, st,
                     static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
                     static_cast<const typename CacheT::raw*>(k_cache),
                     static_cast<const typename CacheT::raw*>(v_cache), block_tables, max_blocks,
                     num_blocks, context_lens, H_q, H_kv, H_q / H_kv, n_splits, score_scale,
                     v_scale, counters, ws_ml, ws_o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_decode: launch failed: %s", hipGetErrorString(e));
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
         H_q / H_kv <= 16;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t S, int32_t H_q, int32_t H_kv, int32_t D,
                                            int32_t max_context_len) {
  if (S <= 0 || H_q <= 0 || D <= 0) return 0;
  const int64_t n_splits = decode_num_splits(max_context_len);
  return decode_counter_bytes(S, H_kv) +
         static_cast<size_t>(S) * H_q * n_splits * (D + 2) * sizeof(float);
}

extern "C" pa_status pa_decode(void* stream, void* out, pa_dtype out_dt, const void* q,
                               pa_dtype q_dt, const void* k_cache, const void* v_cache,
                               pa_dtype cache_dt, const int32_t* block_tables, int32_t max_blocks,
                               int32_t num_blocks, const int32_t* context_lens, int32_t S,
                               int32_t H_q, int32_t H_kv, int32_t D, int32_t bs,
                               int32_t max_context_len, float sm_scale, float k_scale,
                               float v_scale, void* ws, size_t ws_bytes) {
  if (bs != kBlock) return fail(PA_ERR_INVALID, "pa_decode: block size %d != 16", bs);
  if (S < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return fail(PA_ERR_INVALID, "pa_decode: S=%d H_q=%d H_kv=%d", S, H_q, H_kv);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "pa_decode: D=%d not in {64,128}", D);
  if (max_blocks <= 0 || num_blocks <= 0 || max_context_len <= 0)
    return fail(PA_ERR_INVALID, "pa_decode: max_blocks=%d num_blocks=%d max_context_len=%d",
                max_blocks, num_blocks, max_context_len);
  if (static_cast<int64_t>(max_blocks) * kBlock > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_decode: max_blocks=%d too large", max_blocks);
  const bool f32 = q_dt == PA_F32 && cache_dt == PA_F32 && out_dt == PA_F32;
  const bool bf = q_dt == PA_BF16 && out_dt == PA_BF16 &&
                  (cache_dt == PA_BF16 || cache_dt == PA_FP8_E4M3);
  if (!f32 && !bf)
    return fail(PA_ERR_INVALID, "pa_decode: unsupported dtypes q=%d cache=%d out=%d", q_dt,
                cache_dt, out_dt);
  if (cache_dt == PA_FP8_E4M3 &&
      (!(k_scale > 0.f) || !(v_scale > 0.f) || !__builtin_isfinite(k_scale) ||
       !__builtin_isfinite(v_scale)))
    return fail(PA_ERR_INVALID, "pa_decode: fp8 scales must be finite and > 0");
  if (S == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID, "pa_decode: NULL buffer");
  if (S > 65535 || H_kv > 65535)
    return fail(PA_ERR_INVALID, "pa_decode: S=%d or H_kv=%d exceeds grid limits", S, H_kv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (decode_uses_mfma(q_dt, cache_dt, H_q, H_kv)) {
    const size_t need = pa_decode_workspace_bytes(S, H_q, H_kv, D, max_context_len);
    if (!ws || ws_bytes < need)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace %zu bytes < %zu required", ws_bytes,
                  need);
    if (cache_dt == PA_BF16) {
      if (D == 128)
        return launch_decode_mfma<BF16, 128>(st, out, q, k_cache, v_cache, block_tables,
                                             max_blocks, num_blocks, context_lens, S, H_q, H_kv,
                                             max_context_len, sm_scale, 1.f, 1.f, ws);
      return launch_decode_mfma<BF16, 64>(st, out, q, k_cache, v_cache, block_tables, max_blocks,
                                          num_blocks, context_lens, S, H_q, H_kv, max_context_len,
                                          sm_scale, 1.f, 1.f, ws);
    }
    if (D == 128)
      return launch_decode_mfma<FP8, 128>(st, out, q, k_cache, v_cache, block_tables, max_blocks,
                                          num_blocks, context_lens, S, H_q, H_kv, max_context_len,
                                          sm_scale, k_scale, v_scale, ws);
    return launch_decode_mfma<FP8, 64>(st, out, q, k_cache, v_cache, block_tables, max_blocks,
                                       num_blocks, context_lens, S, H_q, H_kv, max_context_len,
                                       sm_scale, k_scale, v_scale, ws);
  }
  return launch_attend_generic(st, out, out_dt, q, q_dt, k_cache, v_cache, cache_dt, block_tables,
                               max_blocks, num_blocks, context_lens, nullptr, nullptr, 0, S, H_q,
                               H_kv, D, sm_scale, k_scale, v_scale);
}
