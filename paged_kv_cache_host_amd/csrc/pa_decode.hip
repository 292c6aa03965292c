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
#include "pa_device.h"
#include "pa_internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace pa {

constexpr int kDecodeWaves = 8;                  // waves per work-group
constexpr int kMinChunkShift = 7;               // smallest chunk: 128 blocks = 2048 tokens
constexpr int kMaxChunkShift = 9;               // largest chunk: 512 blocks = 8192 tokens
constexpr int kMaxGroup = 16;                    // query heads per KV head (MFMA columns)
constexpr int kMaxSeqsPerLaunch = 4096;          // item prefix kept in LDS
constexpr int kThreads = kWave * kDecodeWaves;

// Chunk size (log2 of the blocks one work item covers), a function of the
// launch shape only.  Small chunks spread a few long contexts over the chip;
// once the launch's KV rows (bounded by S x H_kv x max_context_len) fill
// two chip-fulls (2 x 256 CUs) of items at a larger size, the larger size
// wins: fewer items carry less per-item set-up and fewer partials to merge.
inline int32_t decode_chunk_shift(int32_t S, int32_t H_kv, int32_t max_context_len) {
  const int64_t work = static_cast<int64_t>(S) * H_kv * max_context_len;
  for (int32_t sh = kMaxChunkShift; sh > kMinChunkShift; --sh)
    if (work >= 2 * 256 * (int64_t{kBlock} << sh)) return sh;
  return kMinChunkShift;
}

inline int32_t decode_num_chunks(int32_t max_context_len, int32_t shift) {
  const int32_t nblk = (max_context_len + kBlock - 1) / kBlock;
  return nblk <= 0 ? 1 : ((nblk - 1) >> shift) + 1;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// First dim of the 8 that lane group g feeds to score MFMA step s (the same
// map is used for K and Q, so any consistent choice gives q.k).
//   bf16: chunk (4s + g) of 8 dims;
//   fp8:  16-dim chunk (g + 4 * (s/2)), half (s % 2).
template <typename CacheT>
__device__ __forceinline__ int kdim(int s, int g) {
  if constexpr (sizeof(typename CacheT::raw) == 1)
    return 16 * (g + 4 * (s >> 1)) + 8 * (s & 1);
  else
    return 32 * s + 8 * g;
}

template <typename CacheT, int D>
struct BlockRegs;

template <int D>
struct BlockRegs<BF16, D> {
  u32x4 k[D / 32];  // one 16-byte chunk per score step
  u32x2 v[D / 16];  // 4 tokens of one dim per 16-dim slice
};

template <int D>
struct BlockRegs<FP8, D> {
  u32x4 k[D / 64];  // one 16-byte chunk per two score steps
  uint32_t v[D / 16];
};

// Loads 16-token sub-block j of a sequence (tokens 16 j .. 16 j + 15) from a
// cache of BS-token blocks (BS = 8, 16 or 32): K [blocks][H_kv][D/x][BS][x],
// V [blocks][H_kv][D][BS].  With BS = 32 the sub-block is one half of block
// j / 2; with BS = 8 its K rows and V quads come from blocks 2 j and
// 2 j + 1 (lane by lane).  Table indices are clamped to the last of the
// sequence's nphys blocks and every entry into the pool.
template <typename CacheT, int D, int BS>
__device__ __forceinline__ void load_block(BlockRegs<CacheT, D>& r,
                                           const typename CacheT::raw* __restrict__ k_cache,
                                           const typename CacheT::raw* __restrict__ v_cache,
                                           const int32_t* __restrict__ table, int32_t j,
                                           int32_t nphys, int32_t num_blocks, int32_t H_kv,
                                           int32_t kvh, int c, int g) {
  using R = typename CacheT::raw;
  constexpr int X = 16 / sizeof(R);
  const R* kt;
  const R* vt;
  if constexpr (BS >= kBlock) {
    constexpr int kSubs = BS / kBlock;       // sub-blocks per block
    const int64_t tile =
        static_cast<int64_t>(safe_block(table[min(j / kSubs, nphys - 1)], num_blocks)) * H_kv + kvh;
    const int tok0 = kBlock * (j % kSubs);   // first token of the sub-block in its block
    kt = k_cache + tile * (BS * D) + (tok0 + c) * X;
    vt = v_cache + tile * (BS * D) + c * BS + tok0 + 4 * g;
  } else {
    static_assert(kBlock % BS == 0, "block size divides 16");
    constexpr int kPer = kBlock / BS;        // blocks per sub-block
    const int64_t tk =
        static_cast<int64_t>(safe_block(table[min(kPer * j + c / BS, nphys - 1)], num_blocks)) *
            H_kv + kvh;
    const int64_t tv =
        static_cast<int64_t>(safe_block(table[min(kPer * j + (4 * g) / BS, nphys - 1)],
                                        num_blocks)) * H_kv + kvh;
    kt = k_cache + tk * (BS * D) + (c % BS) * X;
    vt = v_cache + tv * (BS * D) + c * BS + (4 * g) % BS;
  }
  if constexpr (sizeof(R) == 2) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      r.k[s] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kt + (4 * s + g) * BS * X));
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      // with 32-token blocks a sub-block's values are half of each 64-byte
      // row; the other half follows in the step's second load, so those rows
      // are kept in cache
      if constexpr (BS > kBlock)
        r.v[t] = *reinterpret_cast<const u32x2*>(vt + 16 * t * BS);
      else
        r.v[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vt + 16 * t * BS));
    }
  } else {
#pragma unroll
    for (int s = 0; s < D / 64; ++s)
      r.k[s] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kt + (g + 4 * s) * BS * X));
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      if constexpr (BS > kBlock)
        r.v[t] = *reinterpret_cast<const uint32_t*>(vt + 16 * t * BS);
      else
        r.v[t] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vt + 16 * t * BS));
    }
  }
}

template <typename CacheT, int D>
__device__ __forceinline__ bf16x8 k_operand(const BlockRegs<CacheT, D>& r, int s) {
  if constexpr (sizeof(typename CacheT::raw) == 2) {
    return __builtin_bit_cast(bf16x8, r.k[s]);
  } else {
    const u32x4 w = r.k[s >> 1];
    u32x2 half;
    half[0] = (s & 1) ? w[2] : w[0];
    half[1] = (s & 1) ? w[3] : w[1];
    return fp8x8_to_bf16x8(half);
  }
}

template <typename CacheT, int D>
__device__ __forceinline__ bf16x4 v_operand(const BlockRegs<CacheT, D>& r, int t) {
  if constexpr (sizeof(typename CacheT::raw) == 2) {
    return __builtin_bit_cast(bf16x4, r.v[t]);
  } else {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[t], 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.v[t], 1.0f, true);
    bf16x4 o;
    o[0] = lo[0];
    o[1] = lo[1];
    o[2] = hi[0];
    o[3] = hi[1];
    return o;
  }
}

template <typename OutT>
__device__ __forceinline__ void store_out4(typename OutT::raw* dst, f32x4 v) {
  if constexpr (sizeof(typename OutT::raw) == 2) {
    u32x2 w;
    w[0] = static_cast<uint32_t>(f32_to_bf16(v[0])) |
           (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    w[1] = static_cast<uint32_t>(f32_to_bf16(v[2])) |
           (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<u32x2*>(dst) = w;
  } else {
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

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
  __shared__ float lds_o[kDecodeWaves][kMaxGroup][D];
  __shared__ float lds_ml[kDecodeWaves][kMaxGroup][2];
  __shared__ int32_t pre[kMaxSeqsPerLaunch + 1];     // full-chunk items before seq i
  __shared__ int32_t order[kMaxSeqsPerLaunch];       // sequences with a partial chunk
  __shared__ int32_t key_s[kThreads];
  __shared__ int32_t wave_sums[kDecodeWaves];
  __shared__ int32_t s_item;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c = lane & 15;
  const int g = lane >> 4;

  // Work items, largest first: every full chunk (2^chunk_shift blocks; the
  // last chunk index also takes any excess past max_context_len), then the
  // partial last chunk of each sequence, in decreasing size, so that the
  // queue ends with its smallest items.
  auto blocks_of = [&](int32_t i) -> int32_t {
    const int32_t Li = min(context_lens[i], max_blocks * BS);
    return Li <= 0 ? 0 : (Li + kBlock - 1) / kBlock;
  };
  auto full_of = [&](int32_t nb) -> int32_t { return min(nb >> chunk_shift, n_chunks); };
  auto part_of = [&](int32_t nb) -> int32_t {
    const int32_t f = full_of(nb);
    return (f < n_chunks && nb > (f << chunk_shift)) ? nb - (f << chunk_shift) : 0;
  };
  // block-wide exclusive scan of v over the launch's sequences, kThreads at
  // a time; returns this thread's exclusive prefix and updates carry
  auto scan = [&](int32_t v, int32_t& carry) -> int32_t {
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    int32_t before = carry, tot = 0;
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (w < wave) before += wave_sums[w];
      tot += wave_sums[w];
    }
    carry += tot;
    __syncthreads();
    return before + x - v;
  };
  // the first ticket is requested before the item list is built, so that
  // the atomic's latency overlaps it
  int32_t next = 0;
  if (tid == 0) next = atomicAdd(&counters[0], 1);
  int32_t total_full = 0, n_part = 0;
  for (int32_t base = 0; base < S; base += kThreads) {
    const int32_t i = base + tid;
    const int32_t nb = i < S ? blocks_of(i) : 0;
    const int32_t full = H_kv * full_of(nb);
    const int32_t has_part = part_of(nb) > 0 ? 1 : 0;
    const int32_t e_full = scan(full, total_full);
    const int32_t e_part = scan(has_part, n_part);
    if (i < S) {
      pre[i] = e_full;
      if (has_part) order[e_part] = i;  // index order; re-sorted below when small
    }
  }
  if (tid == 0) pre[S] = total_full;
  if (S <= kThreads) {
    // deterministic sort of the partial chunks by size, descending, ties in
    // sequence order: rank = #larger + #equal with a smaller index
    const int32_t my = tid < S ? part_of(blocks_of(tid)) : 0;
    key_s[tid] = my;
    __syncthreads();
    int32_t rank = 0;
    if (my > 0) {
      for (int32_t j = 0; j < S; ++j) {
        const int32_t kj = key_s[j];
        rank += (kj > my) || (kj == my && j < tid);
      }
    }
    __syncthreads();
    if (my > 0) order[rank] = tid;
  }
  __syncthreads();
  const int32_t total = total_full + n_part * H_kv;

  while (true) {
    if (tid == 0) s_item = next;
    __syncthreads();
    const int32_t item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= total) break;
    int32_t seq_, chunk_, kvh_;
    if (item < total_full) {
      // last seq with pre[seq] <= item
      int32_t lo = 0, hi = S - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= item)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int32_t r = item - pre[lo];
      seq_ = lo;
      chunk_ = r / H_kv;
      kvh_ = r % H_kv;
    } else {
      const int32_t u = item - total_full;
      seq_ = order[u / H_kv];
      kvh_ = u % H_kv;
      chunk_ = full_of(blocks_of(seq_));
    }
    const int seq = __builtin_amdgcn_readfirstlane(seq_);
    const int chunk = __builtin_amdgcn_readfirstlane(chunk_);
    const int kvh = __builtin_amdgcn_readfirstlane(kvh_);
    const int32_t n_valid = full_of(blocks_of(seq)) + (part_of(blocks_of(seq)) > 0 ? 1 : 0);

  const int32_t L = min(context_lens[seq], max_blocks * BS);
  const int32_t nblk = (L + kBlock - 1) / kBlock;     // 16-token sub-blocks
  const int32_t nphys = (L + BS - 1) / BS;            // table entries in use
  const int32_t c0 = chunk << chunk_shift;
  const int32_t b1 = (chunk == n_chunks - 1) ? nblk : min(nblk, c0 + (1 << chunk_shift));
  const int32_t* __restrict__ table = block_tables + static_cast<int64_t>(seq) * max_blocks;

  // Q^T operand: column c = head kvh*G + c, zero for padded columns.
  bf16x8 qb[D / 32];
  {
    const bool live = c < G;
    const uint16_t* qp = q + (static_cast<int64_t>(seq) * H_q + kvh * G + (live ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + kdim<CacheT>(s, g));
      qb[s] = live ? v : bf16x8{};
    }
  }

  f32x4 o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;


  // One step: blocks p and p+1 (the second is absent when p+1 == b1; its
  // loads then repeat block p's and all its positions are masked).
  //
  // Softmax reference: weights are exp2(score - m_run) with a reference
  // m_run that is only raised when some score of the step exceeds it by more
  // than kLazy (log2 units).  Softmax does not depend on the reference, so
  // the result is unchanged up to rounding, while every weight stays below
  // 2^kLazy; most steps then need neither the cross-lane max nor a rescale of
  // the accumulators.
  constexpr float kLazy = 8.0f;
  auto compute = [&](const BlockRegs<CacheT, D>& ra, const BlockRegs<CacheT, D>& rb, int32_t p) {
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      sa = mfma16x16x32(k_operand(ra, s), qb[s], sa);
      sb = mfma16x16x32(k_operand(rb, s), qb[s], sb);
    }
    const int32_t pa_ = p * kBlock + 4 * g;
    const int32_t pb_ = pa_ + kBlock;
    const bool tail = (p + 2) * kBlock > L;  // wave-uniform
    float sc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = sa[j];
      sc[j + 4] = sb[j];
    }
    if (tail) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = (pa_ + j < L) ? sc[j] : -__builtin_inff();
        sc[j + 4] = (pb_ + j < L) ? sc[j + 4] : -__builtin_inff();
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx *= score_scale;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) o[t] *= alpha;
      m_run = m_new;
    }
    // weights as a sum of two bf16 (high part + rounded remainder): about 16
    // significant bits, so that contexts of a few tokens, where one or two
    // weights dominate, keep the output within tolerance
    bf16x4 pa4, pb4, pa4l, pb4l;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ea = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j], score_scale, -m_run));
      const float eb = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j + 4], score_scale, -m_run));
      psum += ea + eb;
      pa4[j] = static_cast<__bf16>(ea);
      pb4[j] = static_cast<__bf16>(eb);
      pa4l[j] = static_cast<__bf16>(ea - static_cast<float>(pa4[j]));
      pb4l[j] = static_cast<__bf16>(eb - static_cast<float>(pb4[j]));
    }
    l_run += psum;
    if (tail) {
      // positions past the context carry zero weight; their stored values
      // may be anything (a reused block), so they are zeroed in the operand
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        bf16x4 va = v_operand(ra, t), vb = v_operand(rb, t);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          va[j] = (pa_ + j < L) ? va[j] : static_cast<__bf16>(0.f);
          vb[j] = (pb_ + j < L) ? vb[j] : static_cast<__bf16>(0.f);
        }
        o[t] = mfma16x16x16(va, pa4, o[t]);
        o[t] = mfma16x16x16(vb, pb4, o[t]);
        o[t] = mfma16x16x16(va, pa4l, o[t]);
        o[t] = mfma16x16x16(vb, pb4l, o[t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x4 va = v_operand(ra, t), vb = v_operand(rb, t);
        o[t] = mfma16x16x16(va, pa4, o[t]);
        o[t] = mfma16x16x16(vb, pb4, o[t]);
        o[t] = mfma16x16x16(va, pa4l, o[t]);
        o[t] = mfma16x16x16(vb, pb4l, o[t]);
      }
    }
  };

  // Wave w takes the chunk's 2-block steps w, w + W, ...  (a fixed
  // assignment keeps the result independent of timing: runs are
  // bit-identical).  The second block's table entry is read at a clamped
  // index (always in range) so that no load sits behind a branch.
  const int32_t n_steps = (b1 - c0 + 1) / 2;
  for (int32_t st = wave; st < n_steps; st += kDecodeWaves) {
    const int32_t p = c0 + 2 * st;
    BlockRegs<CacheT, D> xa, xb;
    load_block<CacheT, D, BS>(xa, k_cache, v_cache, table, p, nphys, num_blocks, H_kv, kvh, c, g);
    load_block<CacheT, D, BS>(xb, k_cache, v_cache, table, min(p + 1, b1 - 1), nphys, num_blocks,
                              H_kv, kvh, c, g);
    compute(xa, xb, p);
  }

  // the next ticket is taken once this item's streaming is done, so that a
  // work-group that runs ahead takes the next item and the queue balances
  // (taking it earlier would bind it to this work-group behind a long item)
  if (tid == 0) next = atomicAdd(&counters[0], 1);
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  // lane (c, g) holds o^T[d = 16t + 4g + r][head c]; a wave without steps
  // holds m = -inf, l = 0, o = 0
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    *reinterpret_cast<f32x4*>(&lds_o[wave][c][16 * t + 4 * g]) = o[t];
  if (g == 0) {
    lds_ml[wave][c][0] = m_run;
    lds_ml[wave][c][1] = l_run;
  }
  __syncthreads();
  // merge the waves: thread -> (head h, 4 consecutive dims)
  constexpr int kPerHead = D / 4;
  for (int item = threadIdx.x; item < G * kPerHead; item += kWave * kDecodeWaves) {
    const int h = item / kPerHead;
    const int d0 = 4 * (item % kPerHead);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, lds_ml[w][h][0]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(lds_ml[w][h][0] - M);
      tot += wt * lds_ml[w][h][1];
      acc += wt * *reinterpret_cast<const f32x4*>(&lds_o[w][h][d0]);
    }
    const int64_t head_row = static_cast<int64_t>(seq) * H_q + kvh * G + h;
    if (n_valid == 1) {
      store_out4<BF16>(out + head_row * D + d0, acc * (out_scale / tot));
    } else {
      const int64_t part = head_row * n_chunks + chunk;
      *reinterpret_cast<f32x4*>(ws_o + part * D + d0) = acc;
      if (d0 == 0) {
        ws_ml[part * 2 + 0] = M;
        ws_ml[part * 2 + 1] = tot;
      }
    }
  }
  __syncthreads();  // LDS reads done before the next item overwrites it
  }
  // the last work-group out resets the counters for the next call
  if (tid == 0) {
    const int32_t done = atomicAdd(&counters[1], 1);
    if (done == static_cast<int32_t>(gridDim.x) - 1) {
      atomicExch(&counters[0], 0);
      atomicExch(&counters[1], 0);
    }
  }
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
  const float* ml = ws_ml + idx * n_chunks * 2;
  const float* po = ws_o + idx * n_chunks * D;
  float M = -__builtin_inff();
  for (int j = 0; j < nsp; ++j) M = fmaxf(M, ml[2 * j]);
  float tot = 0.f;
  float acc[D / kWave];
#pragma unroll
  for (int i = 0; i < D / kWave; ++i) acc[i] = 0.f;
  for (int j = 0; j < nsp; ++j) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * j] - M);
    tot += w * ml[2 * j + 1];
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) acc[i] += w * po[j * D + lane + kWave * i];
  }
  const float inv = nsp ? out_scale / tot : 0.f;
#pragma unroll
  for (int i = 0; i < D / kWave; ++i) out[idx * D + lane + kWave * i] = f32_to_bf16(acc[i] * inv);
}

inline int32_t decode_num_batches(int32_t S) {
  return (S + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch;
}

// Bytes of ticket counters at the front of the workspace (two int32 per
// launch batch of up to kMaxSeqsPerLaunch sequences).
inline size_t decode_counter_bytes(int32_t S) {
  return (static_cast<size_t>(decode_num_batches(S)) * 2 * sizeof(int32_t) + 255) &
         ~static_cast<size_t>(255);
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
  if (n_chunks > 1) {
    const int64_t rows = static_cast<int64_t>(S) * H_q;
    hipError_t e = launch(kDecodeMerge, decode_merge_kernel<D>, dim3((rows + 3) / 4), dim3(256), 0,
                          st, static_cast<uint16_t*>(out), ws_ml, ws_o, context_lens, max_blocks,
                          BS, S, H_q, n_chunks, shift, v_scale);
    if (e != hipSuccess)
      return fail(PA_ERR_DEVICE, "pa_decode: merge launch failed: %s", hipGetErrorString(e));
  }
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
