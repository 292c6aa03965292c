// Device code of decode attention: block loads, the persistent work-group
// body and the chunk merge.  Shared by the decode launch (pa_decode.hip)
// and the fused decode + prefill launch (pa_varlen.hip); the algorithm is
// described at the top of pa_decode.hip.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

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

inline int32_t decode_num_batches(int32_t S) {
  return (S + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch;
}

// Bytes of ticket counters at the front of the decode workspace (two int32
// per launch batch of up to kMaxSeqsPerLaunch sequences, rounded up to 256
// bytes; the fused append + decode launch keeps a third word there).
inline size_t decode_counter_bytes(int32_t S) {
  return (static_cast<size_t>(decode_num_batches(S)) * 2 * sizeof(int32_t) + 255) &
         ~static_cast<size_t>(255);
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
// kOverride (the fused append + decode launch, BS = 16): table entry
// `last_ti` (when >= 0) is taken as `last_blk` instead of being read (the
// launch itself enters that block into the table).
template <typename CacheT, int D, int BS, bool kOverride = false>
__device__ __forceinline__ void load_block(BlockRegs<CacheT, D>& r,
                                           const typename CacheT::raw* __restrict__ k_cache,
                                           const typename CacheT::raw* __restrict__ v_cache,
                                           const int32_t* __restrict__ table, int32_t j,
                                           int32_t nphys, int32_t num_blocks, int32_t H_kv,
                                           int32_t kvh, int c, int g, int32_t last_ti = -1,
                                           int32_t last_blk = 0) {
  using R = typename CacheT::raw;
  constexpr int X = 16 / sizeof(R);
  const R* kt;
  const R* vt;
  if constexpr (BS >= kBlock) {
    constexpr int kSubs = BS / kBlock;       // sub-blocks per block
    const int32_t ti = min(j / kSubs, nphys - 1);
    int32_t e;
    if constexpr (kOverride) {
      // read as constant memory so that the entry is a scalar load, as in the
      // plain launch: the entries this launch writes are never taken from
      // the table (ti == last_ti takes last_blk)
      using ConstI32 = const __attribute__((address_space(4))) int32_t;
      const int32_t loaded = ((ConstI32*)table)[ti];
      e = ti == last_ti ? last_blk : loaded;
    } else {
      e = table[ti];
    }
    const int64_t tile = static_cast<int64_t>(safe_block(e, num_blocks)) * H_kv + kvh;
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

// LDS of the decode work-group.
template <int D>
struct DecodeShared {
  // small fields first: their addresses fit the LDS instructions' offsets
  int32_t s_item;
  int32_t s_flag;
  int32_t wave_sums[kDecodeWaves];
  float ml[kDecodeWaves][kMaxGroup][2]; // per-wave (m, l)
  int32_t key_s[kThreads];
  int32_t pre[kMaxSeqsPerLaunch + 1];   // full-chunk items before seq i
  int32_t order[kMaxSeqsPerLaunch];     // sequences with a partial chunk
  alignas(16) float o[kDecodeWaves][kMaxGroup][D];  // per-wave unnormalised outputs
};

// Merges the nsp chunk partials of one (sequence, query head) row idx: one
// wave, D / 64 dimensions per lane.  ws_ml[2 (idx n_chunks + j)] = (m, l)
// and ws_o[(idx n_chunks + j) D ..] = unnormalised output of chunk j.
template <int D>
__device__ __forceinline__ void decode_merge_row(uint16_t* __restrict__ out,
                                                 const float* __restrict__ ws_ml,
                                                 const float* __restrict__ ws_o, int64_t idx,
                                                 int nsp, int32_t n_chunks, int lane,
                                                 float out_scale) {
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

// The fused append + decode launch (pa_decode_step): sequence i's new token
// (bf16 K/V rows [S][H_kv][D], flat slot slots[i], position
// context_lens[i] - 1) is written into the cache by the work item that
// attends that position, for its KV head, and the KV-head-0 item enters the
// slot's block into row i of the block tables.
template <typename CacheT>
struct DecodeAppend {
  const int32_t* slots = nullptr;
  const uint16_t* k_new = nullptr;
  const uint16_t* v_new = nullptr;
  typename CacheT::raw* k_cache = nullptr;
  typename CacheT::raw* v_cache = nullptr;
  int32_t* tables = nullptr;
  float k_inv = 1.f, v_inv = 1.f;  // fp8: reciprocal scales
};

template <typename CacheT>
__device__ __forceinline__ typename CacheT::raw encode_new(uint16_t x, float inv) {
  if constexpr (sizeof(typename CacheT::raw) == 1)
    return f32_to_e4m3_sat(bf16_to_f32(x) * inv);
  else
    return x;
}

// One wave's share of a new token: lane l holds dims l*E .. l*E + E - 1
// (E = D / 64) of the token's K row and V row, bf16, packed in kw and vw.
template <int D>
__device__ __forceinline__ void load_new_token(const uint16_t* __restrict__ k_new,
                                               const uint16_t* __restrict__ v_new, int64_t row,
                                               int lane, uint32_t& kw, uint32_t& vw) {
  if constexpr (D == 128) {
    kw = *reinterpret_cast<const uint32_t*>(k_new + row * D + 2 * lane);
    vw = *reinterpret_cast<const uint32_t*>(v_new + row * D + 2 * lane);
  } else {
    kw = k_new[row * D + lane];
    vw = v_new[row * D + lane];
  }
}

// Stores the wave's share of a new token into slot `off` of cache tile
// `tile` (= block * H_kv + KV head): K [D/x][16][x], V [D][16].
template <typename CacheT, int D>
__device__ __forceinline__ void store_new_token(const DecodeAppend<CacheT>& ap, int64_t tile,
                                                int off, int lane, uint32_t kw, uint32_t vw) {
  using CR = typename CacheT::raw;
  constexpr int X = 16 / sizeof(CR);
  constexpr int NCH = D / X;
  constexpr int E = D / kWave;
  const int d = E * lane;
  CR* kd = ap.k_cache + ((tile * NCH + d / X) * kBlock + off) * X + d % X;
  CR* vd = ap.v_cache + (tile * D + d) * kBlock + off;
  if constexpr (E == 2) {
    const CR k0 = encode_new<CacheT>(static_cast<uint16_t>(kw), ap.k_inv);
    const CR k1 = encode_new<CacheT>(static_cast<uint16_t>(kw >> 16), ap.k_inv);
    if constexpr (sizeof(CR) == 2)
      *reinterpret_cast<uint32_t*>(kd) = static_cast<uint32_t>(k0) | (static_cast<uint32_t>(k1) << 16);
    else
      *reinterpret_cast<uint16_t*>(kd) = static_cast<uint16_t>(k0 | (k1 << 8));
    vd[0] = encode_new<CacheT>(static_cast<uint16_t>(vw), ap.v_inv);
    vd[kBlock] = encode_new<CacheT>(static_cast<uint16_t>(vw >> 16), ap.v_inv);
  } else {
    kd[0] = encode_new<CacheT>(static_cast<uint16_t>(kw), ap.k_inv);
    vd[0] = encode_new<CacheT>(static_cast<uint16_t>(vw), ap.v_inv);
  }
}

// Persistent work-group body (the kernel's comment above describes it).
// kVarlen (the fused decode + prefill launch): a context cut into several
// chunks is merged in-kernel by the last of its chunks to finish
// (merge_counters: one per (sequence, KV head), zero before and after).
template <typename CacheT, int D, int BS, bool kVarlen, bool kAppend = false>
__device__ __attribute__((always_inline)) inline void decode_work(DecodeShared<D>& sh,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const typename CacheT::raw* k_cache, const typename CacheT::raw* v_cache,
    const int32_t* block_tables, int32_t max_blocks, int32_t num_blocks,
    const int32_t* __restrict__ context_lens, int32_t S, int32_t H_q, int32_t H_kv, int32_t G,
    int32_t n_chunks, int32_t chunk_shift, float score_scale, float out_scale,
    int32_t* __restrict__ counters, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    int32_t* __restrict__ merge_counters, const DecodeAppend<CacheT>& ap = {}) {
  static_assert(!kAppend || BS == kBlock, "the fused append takes 16-token blocks");
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
    if (lane == kWave - 1) sh.wave_sums[wave] = x;
    __syncthreads();
    int32_t before = carry, tot = 0;
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (w < wave) before += sh.wave_sums[w];
      tot += sh.wave_sums[w];
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
      sh.pre[i] = e_full;
      if (has_part) sh.order[e_part] = i;  // index order; re-sorted below when small
    }
  }
  if (tid == 0) sh.pre[S] = total_full;
  if (S <= kThreads) {
    // deterministic sort of the partial chunks by size, descending, ties in
    // sequence order: rank = #larger + #equal with a smaller index
    const int32_t my = tid < S ? part_of(blocks_of(tid)) : 0;
    sh.key_s[tid] = my;
    __syncthreads();
    int32_t rank = 0;
    if (my > 0) {
      for (int32_t j = 0; j < S; ++j) {
        const int32_t kj = sh.key_s[j];
        rank += (kj > my) || (kj == my && j < tid);
      }
    }
    __syncthreads();
    if (my > 0) sh.order[rank] = tid;
  }
  __syncthreads();
  const int32_t total = total_full + n_part * H_kv;

  while (true) {
    if (tid == 0) sh.s_item = next;
    __syncthreads();
    const int32_t item = __builtin_amdgcn_readfirstlane(sh.s_item);
    if (item >= total) break;
    int32_t seq_, chunk_, kvh_;
    if (item < total_full) {
      // last seq with pre[seq] <= item
      int32_t lo = 0, hi = S - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (sh.pre[mid] <= item)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int32_t r = item - sh.pre[lo];
      seq_ = lo;
      chunk_ = r / H_kv;
      kvh_ = r % H_kv;
    } else {
      const int32_t u = item - total_full;
      seq_ = sh.order[u / H_kv];
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
  // (no __restrict__ on the cache and table pointers: the fused append
  // writes through other pointers to the same memory)
  const int32_t* table = block_tables + static_cast<int64_t>(seq) * max_blocks;

  // fused append: the item that holds position L - 1 (its last chunk)
  // writes the new token.  Only the wave with the item's last step reads
  // that position's block (no other step's pair reaches block b1 - 1), so
  // that wave alone stores the token's K/V, just before the step's loads:
  // its own later loads of the same addresses see the stores, and no other
  // wave waits.  The token's rows and its slot are loaded here and used
  // only at that step (the slot decides the block, which that step takes
  // from the slot instead of the table); the KV-head-0 item enters the block
  // into the table once the item is done.
  int32_t last_ti = -1, app_slot = -1;
  bool app_item = false;
  uint32_t app_k = 0, app_v = 0;
  if constexpr (kAppend) {
    const int32_t raw = context_lens[seq];
    if (chunk == n_valid - 1 && raw >= 1 && raw <= max_blocks * kBlock) {
      app_item = true;
      last_ti = (raw - 1) / kBlock;
      app_slot = ap.slots[seq];
      if (wave == ((b1 - c0 + 1) / 2 - 1) % kDecodeWaves)
        load_new_token<D>(ap.k_new, ap.v_new, static_cast<int64_t>(seq) * H_kv + kvh, lane,
                          app_k, app_v);
    }
  }

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
    int32_t ov_ti = -1, ov_blk = 0;  // table entry taken from the slot at this step
    if constexpr (kAppend) {
      if (app_item && st == n_steps - 1) {
        const int32_t sl = __builtin_amdgcn_readfirstlane(app_slot);
        if (sl >= 0 && sl < num_blocks * kBlock) {
          ov_ti = last_ti;
          ov_blk = sl / kBlock;
          store_new_token<CacheT, D>(ap, static_cast<int64_t>(ov_blk) * H_kv + kvh, sl % kBlock,
                                     lane, app_k, app_v);
          // keeps the compiler from moving this step's cache loads above
          // the stores (the loads go through another pointer)
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
      }
    }
    BlockRegs<CacheT, D> xa, xb;
    load_block<CacheT, D, BS, kAppend>(xa, k_cache, v_cache, table, p, nphys, num_blocks, H_kv,
                                       kvh, c, g, ov_ti, ov_blk);
    load_block<CacheT, D, BS, kAppend>(xb, k_cache, v_cache, table, min(p + 1, b1 - 1), nphys,
                                       num_blocks, H_kv, kvh, c, g, ov_ti, ov_blk);
    compute(xa, xb, p);
  }

  // the next ticket is taken once this item's streaming is done, so that a
  // work-group that runs ahead takes the next item and the queue balances
  // (taking it earlier would bind it to this work-group behind a long item)
  if (tid == 0) next = atomicAdd(&counters[0], 1);
  if constexpr (kAppend) {
    if (app_item && kvh == 0 && tid == 0 && app_slot >= 0 && app_slot < num_blocks * kBlock)
      ap.tables[static_cast<int64_t>(seq) * max_blocks + last_ti] = app_slot / kBlock;
  }
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  // lane (c, g) holds o^T[d = 16t + 4g + r][head c]; a wave without steps
  // holds m = -inf, l = 0, o = 0
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    *reinterpret_cast<f32x4*>(&sh.o[wave][c][16 * t + 4 * g]) = o[t];
  if (g == 0) {
    sh.ml[wave][c][0] = m_run;
    sh.ml[wave][c][1] = l_run;
  }
  __syncthreads();
  // merge the waves: thread -> (head h, 4 consecutive dims)
  constexpr int kPerHead = D / 4;
  for (int item = threadIdx.x; item < G * kPerHead; item += kWave * kDecodeWaves) {
    const int h = item / kPerHead;
    const int d0 = 4 * (item % kPerHead);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sh.ml[w][h][0]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sh.ml[w][h][0] - M);
      tot += wt * sh.ml[w][h][1];
      acc += wt * *reinterpret_cast<const f32x4*>(&sh.o[w][h][d0]);
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
  if constexpr (kVarlen) {
    // the last of a (sequence, KV head)'s n_valid chunks to finish merges
    // their partials: published by every wave's stores, the barrier and
    // one agent-scope release by thread 0 (the counter bump); the
    // work-group completing the count acquires at agent scope before the
    // barrier that lets its waves read them
    if (n_valid > 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  }
  __syncthreads();  // LDS reads done before the next item overwrites it
  if constexpr (kVarlen) {
    if (n_valid > 1) {
      if (tid == 0) {
        const int64_t gi = static_cast<int64_t>(seq) * H_kv + kvh;
        const int32_t prev = __hip_atomic_fetch_add(&merge_counters[gi], 1, __ATOMIC_RELEASE,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        const int32_t last = prev == n_valid - 1;
        if (last) {
          __hip_atomic_store(&merge_counters[gi], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        sh.s_flag = last;
      }
      __syncthreads();
      if (sh.s_flag) {
        for (int h = wave; h < G; h += kDecodeWaves)
          decode_merge_row<D>(out, ws_ml, ws_o, static_cast<int64_t>(seq) * H_q + kvh * G + h,
                              n_valid, n_chunks, lane, out_scale);
      }
    }
  }
  }
}

// The last work-group of a persistent launch to finish resets the ticket
// counters (and any further words of the launch's counter region, up to
// `words`) for the next call.
__device__ __forceinline__ void decode_finish(int32_t* __restrict__ counters, int words = 2) {
  if (threadIdx.x == 0) {
    const int32_t done = atomicAdd(&counters[1], 1);
    if (done == static_cast<int32_t>(gridDim.x) - 1) {
      for (int w = 0; w < words; ++w) atomicExch(&counters[w], 0);
    }
  }
}


}  // namespace pa
