// Device code of the chunked-prefill attention: tile loader, the per
// work-group body and the split-range merge.  Shared by the prefill launch
// (pa_prefill.hip) and the fused decode + prefill launch (pa_varlen.hip);
// the algorithm is described at the top of pa_prefill.hip.
#pragma once

#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPfWaves = 8;                 // waves per work-group
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfRows = 32;                 // query positions per wave
constexpr int kPfKeys = 64;                 // keys per LDS tile (4 blocks)
constexpr int kPfTargetGroups = 256;        // one work-group per compute unit
constexpr int kPfMaxSplit = 8;
constexpr int kPfMinKeysPerSplit = 1024;
constexpr float kPfSafe = 32768.0f;         // bound on a lane's 32 weights of one tile

// LDS bytes of one stage: K [D/8 chunks][64 rows][16 B] + V [D/16][8 chunks][16 dims][16 B].
template <int D>
constexpr int stage_bytes() {
  return D * kPfKeys * 2 * 2;
}

// Position of key `tok` (0..15) of a block among the 16 K rows of that block
// in LDS: the second and third groups of four trade places.
__device__ __forceinline__ int krow_of(int tok) {
  const int quad = tok >> 2;
  const int swapped = (quad == 1 || quad == 2) ? (3 - quad) : quad;
  return (swapped << 2) | (tok & 3);
}

// V in LDS: chunk c (8 keys, 16 B) of dimension d.  The 16 dimensions
// d0..d0+15 of one chunk are 256 contiguous bytes, so the 16 lanes of an
// MFMA operand read that take consecutive dimensions hit distinct banks.
__device__ __forceinline__ int v_off(int d, int c) {
  return (((d >> 4) * (kPfKeys / 8) + c) << 8) + ((d & 15) << 4);
}

struct PfGeom {
  int H_kv, G, hpw, psub, n_head_groups, n_pos_tiles, n_split;
};

// Work split shared by the launcher and the workspace query.
PfGeom pf_geometry(int32_t n_chunks, int32_t max_q_len, int32_t H_q, int32_t H_kv,
                   int32_t max_context_len) {
  PfGeom g;
  g.H_kv = H_kv;
  g.G = H_q / H_kv;
  g.hpw = g.G < kPfWaves ? g.G : kPfWaves;
  g.psub = kPfWaves / g.hpw;
  g.n_head_groups = (g.G + kPfWaves - 1) / kPfWaves;
  const int pos_per_group = kPfRows * g.psub;
  g.n_pos_tiles = (max_q_len + pos_per_group - 1) / pos_per_group;
  const int64_t groups =
      static_cast<int64_t>(n_chunks) * g.n_pos_tiles * H_kv * g.n_head_groups;
  int split = groups > 0 ? static_cast<int>(kPfTargetGroups / groups) : 1;
  const int by_keys = max_context_len / kPfMinKeysPerSplit;
  if (split > by_keys) split = by_keys;
  if (split > kPfMaxSplit) split = kPfMaxSplit;
  if (split < 1) split = 1;
  g.n_split = split;
  return g;
}

// Bytes of one split partial of one (row, head): its output normalised by
// its own weight sum as fp16 (the values are weighted means of V, which the
// kernel already holds in fp16, so the range is V's), then (m, l) as fp32.
inline size_t pf_slot_bytes(int32_t D) {
  return static_cast<size_t>(D) * sizeof(uint16_t) + 2 * sizeof(float);
}

// Bytes of split partials that any launch with at most n_chunks slices of
// at most max_q_len queries (keys up to max_context_len) can need: the
// split count grows as the batch shrinks, so a smaller batch may need more
// than the largest one.  With s splits a batch has at most
// 256 / (s H_kv n_head_groups) slice-tiles of pos_per_group rows.
inline size_t pf_partials_bound(int32_t n_chunks, int32_t max_q_len, int32_t H_q, int32_t H_kv,
                                int32_t D, int32_t max_context_len) {
  const PfGeom g = pf_geometry(n_chunks, max_q_len, H_q, H_kv, max_context_len);
  const int64_t ppg = static_cast<int64_t>(kPfRows) * g.psub;
  const int64_t tiles_max = static_cast<int64_t>(n_chunks) * g.n_pos_tiles;
  const int64_t rows_max = static_cast<int64_t>(n_chunks) * max_q_len;
  int64_t best = 0;  // split x workspace rows
  for (int s = 2; s <= kPfMaxSplit; ++s) {
    if (max_context_len / kPfMinKeysPerSplit < s) break;
    const int64_t tiles = std::min<int64_t>(
        tiles_max, kPfTargetGroups / (static_cast<int64_t>(s) * H_kv * g.n_head_groups));
    if (tiles <= 0) break;
    best = std::max(best, s * std::min(rows_max, tiles * ppg));
  }
  return static_cast<size_t>(best) * H_q * pf_slot_bytes(D);
}


// Moves one 64-key tile (four 16-key sub-blocks x K and V of one KV head)
// from the paged cache into an LDS stage as 16-byte pieces spread over the
// work-group's threads: piece p = wave * 64 + lane + i * threads.  A
// sub-block-head tile has a multiple of 64 pieces, so which tensor and
// sub-block a piece belongs to is the same for the whole wave (scalar), and
// every offset splits into a scalar part and a lane part that does not depend
// on i.  BS is the cache's block size: a 16-key sub-block is one block (16),
// half of one (32: the half at 16 (b & 1) keys), or two (8: its first eight
// keys in one block, the last eight in the next, chosen lane by lane).
template <typename CacheT, int D, int BS>
struct TileLoader {
  using CR = typename CacheT::raw;
  static constexpr int kElems = 16 / sizeof(CR);            // cache elements per piece
  static constexpr int kPerBlock = D * 16 / kElems;        // pieces per (sub-block, head), K or V
  static constexpr int kHalf = 4 * kPerBlock;               // K pieces of a tile
  static constexpr int kPieces = 2 * kHalf;
  static constexpr int NLD = kPieces / kPfThreads;          // pieces per thread
  static_assert(kPieces % kPfThreads == 0, "tile pieces must divide over the threads");
  static_assert(kPerBlock % kWave == 0, "a wave's pieces must share one block");
  static constexpr bool kWide = sizeof(CR) == 1;            // fp8 pieces widen to two chunks
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static constexpr int kX = kElems;                         // K's innermost run (16 bytes)

  int wave;      // scalar
  int lane;
  int k_lane;    // LDS offset, lane part, K pieces
  int v_lane;    // LDS offset, lane part, V pieces
  int v_key;     // first key of the lane's V piece inside its sub-block
  int k_ge;      // cache elements from the wave's first K piece to the lane's
  int v_ge;      // same for V
  bool k_hi;     // 8-key blocks: the lane's K piece is in the sub-block's second block
  bool v_hi;     // same for V (a 16-key fp8 V piece straddles both: not used)

  // The cache holds K as [block][head][D / kX][BS][kX] and V as
  // [block][head][D][BS].  In a sub-block, K piece e = chunk * 16 + key
  // (one key's kX elements of one chunk) and V piece e = dim * 2 + half (8
  // keys of one dimension; fp8: e = dim, all 16 keys).
  __device__ TileLoader(int wave_, int lane_) : wave(wave_), lane(lane_) {
    constexpr int R = BS < 16 ? BS : 16;   // keys of a sub-block inside one block
    int k_key, v_dim, v_half;
    if (!kWide) {
      // Each 16 lanes write 256 contiguous LDS bytes: a lane loads the K
      // key (of the 16 of its chunk) or the V dimension and half whose
      // LDS slot is its own, rather than writing its piece to a scattered
      // slot.  The 16 lanes still read contiguous runs of the cache.
      k_lane = (lane >> 4) * (kPfKeys * 16) + (lane & 15) * 16;
      k_key = krow_of(lane & 15);
      v_lane = (lane >> 5) * 2048 + ((lane >> 4) & 1) * 256 + (lane & 15) * 16;
      v_dim = (lane & 15) + 16 * (lane >> 5);
      v_half = (lane >> 4) & 1;
      v_key = v_half * 8;
    } else {
      k_lane = (lane >> 4) * 2 * (kPfKeys * 16) + krow_of(lane & 15) * 16;
      k_key = lane & 15;
      v_lane = (lane >> 4) * 2048 + (lane & 15) * 16;
      v_dim = lane;
      v_half = 0;
      v_key = 0;
    }
    k_hi = BS == 8 && k_key >= 8;
    v_hi = BS == 8 && !kWide && v_half;
    k_ge = ((lane >> 4) * BS + k_key % R) * kX;
    v_ge = v_dim * BS + (BS == 8 ? 0 : v_half * 8);
  }
  // scalar description of piece i of this wave
  struct Piece {
    bool v;
    int b;      // block of the tile
    int e0;     // index of the wave's first piece inside the (block, head) tile
  };
  __device__ Piece piece(int i) const {
    const int p = wave * kWave + i * kPfThreads;
    Piece q;
    // when the K half is a whole number of sweeps over the threads, which
    // tensor a piece belongs to depends on i alone
    q.v = kHalf % kPfThreads == 0 ? i * kPfThreads >= kHalf : p >= kHalf;
    const int pp = q.v ? p - kHalf : p;
    q.b = pp / kPerBlock;
    q.e0 = pp % kPerBlock;
    return q;
  }

  // Entries of the block table a tile reads: lanes 0..n-1 of `ids` hold
  // them (BS 16: one per sub-block; 32: one per two; 8: two per sub-block).
  static constexpr int kIdsPerTile = kPfKeys / BS;

  // Scalar part of piece q's offset inside its block, in cache elements.
  __device__ static int scalar_off(const Piece& q) {
    const int half = BS == 32 ? (q.b & 1) * 16 : 0;
    if (!q.v) return ((q.e0 >> 4) * BS + half) * kX;
    return (kWide ? q.e0 : q.e0 >> 1) * BS + half;
  }

  // ids: the tile's table entries (see kIdsPerTile), already inside the
  // pool.  Blocks past the context are loaded too (any valid id): their
  // keys lie beyond `valid`, so store() zeroes their V and the causal mask
  // drops their scores.  Loading unconditionally keeps the loads free of
  // any use before the store, so their latency overlaps the tile's compute.
  __device__ void load1(u32x4& r, int i, const CR* __restrict__ k_cache,
                        const CR* __restrict__ v_cache, int32_t ids, int32_t kvh,
                        int32_t H_kv, int32_t num_blocks) const {
    const Piece q = piece(i);
    const CR* cache = q.v ? v_cache : k_cache;
    const int off = scalar_off(q) + (q.v ? v_ge : k_ge);
    if constexpr (BS != 8) {
      const int32_t bk = safe_block(__builtin_amdgcn_readlane(ids, BS == 16 ? q.b : q.b >> 1),
                                    num_blocks);
      const CR* base = cache + (static_cast<int64_t>(bk) * H_kv + kvh) * (D * BS);
      r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
    } else {
      const int32_t b0 = safe_block(__builtin_amdgcn_readlane(ids, 2 * q.b), num_blocks);
      const int32_t b1 = safe_block(__builtin_amdgcn_readlane(ids, 2 * q.b + 1), num_blocks);
      const CR* base0 = cache + (static_cast<int64_t>(b0) * H_kv + kvh) * (D * BS);
      const CR* base1 = cache + (static_cast<int64_t>(b1) * H_kv + kvh) * (D * BS);
      if (kWide && q.v) {
        // 16 keys of one dimension: eight bytes from each block
        const u32x2 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base0 + off));
        const u32x2 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base1 + off));
        r = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        const bool second = q.v ? v_hi : k_hi;
        r = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>((second ? base1 : base0) + off));
      }
    }
  }
  __device__ void load(u32x4* regs, const CR* __restrict__ k_cache, const CR* __restrict__ v_cache,
                       int32_t ids, int32_t kvh, int32_t H_kv, int32_t num_blocks) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i) load1(regs[i], i, k_cache, v_cache, ids, kvh, H_kv, num_blocks);
  }

  // Piece i of the tile into a stage, V beyond the context not cleared.
  __device__ void store1(const u32x4& w0, int i, uint8_t* stage) const {
    const Piece q = piece(i);
    u32x4 w = w0;
    if (!kWide) {
      if (!q.v) {
        const int off = (q.e0 >> 4) * (kPfKeys * 16) + q.b * 16 * 16;
        *reinterpret_cast<u32x4*>(stage + off + k_lane) = w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = bf16x2_to_f16x2(w[j]);
        const int off = D * kPfKeys * 2 + ((q.e0 >> 1) >> 4) * 2048 + 2 * q.b * 256;
        *reinterpret_cast<u32x4*>(stage + off + v_lane) = w;
      }
    } else if (!q.v) {
      const int off = (q.e0 >> 4) * 2 * (kPfKeys * 16) + q.b * 16 * 16 + k_lane;
      *reinterpret_cast<bf16x8*>(stage + off) = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
      *reinterpret_cast<bf16x8*>(stage + off + kPfKeys * 16) = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
    } else {
      const int off = D * kPfKeys * 2 + (q.e0 >> 4) * 2048 + 2 * q.b * 256 + v_lane;
      *reinterpret_cast<f16x8*>(stage + off) = fp8x8_to_f16x8(u32x2{w[0], w[1]});
      *reinterpret_cast<f16x8*>(stage + off + 256) = fp8x8_to_f16x8(u32x2{w[2], w[3]});
    }
  }

  // `valid` = keys of the tile that exist; V beyond them is stored as zero.
  __device__ void store(const u32x4* regs, uint8_t* stage, int valid) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const Piece q = piece(i);
      u32x4 w = regs[i];
      if (!kWide) {
        if (!q.v) {
          // e = chunk * 16 + token
          const int off = (q.e0 >> 4) * (kPfKeys * 16) + q.b * 16 * 16;
          *reinterpret_cast<u32x4*>(stage + off + k_lane) = w;
        } else {
          // e = dim * 2 + half; v_off(dim, 2 b + half)
          if (valid < kPfKeys) {  // last tile of the range only
            const int key0 = q.b * 16 + v_key;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int k = key0 + 2 * j;
              const uint32_t m = (k < valid ? 0xFFFFu : 0u) | (k + 1 < valid ? 0xFFFF0000u : 0u);
              w[j] &= m;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = bf16x2_to_f16x2(w[j]);
          const int off = D * kPfKeys * 2 + ((q.e0 >> 1) >> 4) * 2048 + 2 * q.b * 256;
          *reinterpret_cast<u32x4*>(stage + off + v_lane) = w;
        }
      } else if (!q.v) {
        // e = chunk8 * 16 + token: bf16 chunks 2 chunk8, 2 chunk8 + 1
        const int off = (q.e0 >> 4) * 2 * (kPfKeys * 16) + q.b * 16 * 16 + k_lane;
        *reinterpret_cast<bf16x8*>(stage + off) = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
        *reinterpret_cast<bf16x8*>(stage + off + kPfKeys * 16) = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
      } else {
        // e = dim: tokens 0..7 -> chunk 2 b, 8..15 -> chunk 2 b + 1
        f16x8 v0 = fp8x8_to_f16x8(u32x2{w[0], w[1]});
        f16x8 v1 = fp8x8_to_f16x8(u32x2{w[2], w[3]});
        const int key0 = q.b * 16;
        if (valid < kPfKeys && key0 + 16 > valid) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (key0 + j >= valid) v0[j] = static_cast<_Float16>(0.0f);
            if (key0 + 8 + j >= valid) v1[j] = static_cast<_Float16>(0.0f);
          }
        }
        const int off = D * kPfKeys * 2 + (q.e0 >> 4) * 2048 + 2 * q.b * 256 + v_lane;
        *reinterpret_cast<f16x8*>(stage + off) = v0;
        *reinterpret_cast<f16x8*>(stage + off + 256) = v1;  // chunk 2 b + 1
      }
    }
  }
};

// Merge of the key-range partials of one (row, head) pair, shared by the
// merge kernel and the fused launch's in-kernel merge (same arithmetic, so
// the two give identical bits).  Partial j of the pair sits at
// slot = j * stride + pair: ws_ml[2 slot] = m (base-2 running maximum),
// ws_ml[2 slot + 1] = l (weight sum), ws_o[slot * D ..] = output / l as
// fp16; a partial with l = 0 saw no key and is skipped.  Merged:
//   M = max_j m_j,  W_j = 2^(m_j - M) l_j,  out = sum_j W_j o_j / sum_j W_j.
__device__ __forceinline__ float pf_merge_max(const float* __restrict__ ws_ml, int64_t pair,
                                              int64_t stride, int n_split) {
  float M = -__builtin_inff();
  for (int j = 0; j < n_split; ++j) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * (j * stride + pair));
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  return M;
}

__device__ __forceinline__ float pf_merge_weight(float m, float l, float M) {
  return __builtin_amdgcn_exp2f(m - M) * l;
}

// v_scale / (sum of the partials' weights W_j), or 0 if none
__device__ __forceinline__ float pf_merge_inv(const float* __restrict__ ws_ml, int64_t pair,
                                              int64_t stride, int n_split, float M,
                                              float v_scale) {
  float L = 0.f;
  for (int j = 0; j < n_split; ++j) {
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * (j * stride + pair));
    if (!(ml.y > 0.f)) continue;
    L += pf_merge_weight(ml.x, ml.y, M);
  }
  return L > 0.f ? v_scale / L : 0.f;
}

// 4 normalised partial values as stored (fp16, round to nearest even), and
// back (exact)
__device__ __forceinline__ u32x2 pf_pack_f16x4(const f32x4& v) {
  u32x2 w;
  w[0] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[0]))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[1]))) << 16);
  w[1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2]))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[3]))) << 16);
  return w;
}

__device__ __forceinline__ f32x4 pf_unpack_f16x4(u32x2 w) {
  return f32x4{static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[0]))),
               static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[0] >> 16))),
               static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[1]))),
               static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[1] >> 16)))};
}

// dimensions d0 .. d0 + 3 of sum_j W_j o_j
template <int D>
__device__ __forceinline__ f32x4 pf_merge_dims4(const float* __restrict__ ws_ml,
                                                const uint16_t* __restrict__ ws_o, int64_t pair,
                                                int64_t stride, int n_split, float M, int d0) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n_split; ++j) {
    const int64_t slot = j * stride + pair;
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * slot);
    if (!(ml.y > 0.f)) continue;
    const float w = pf_merge_weight(ml.x, ml.y, M);
    acc += w * pf_unpack_f16x4(*reinterpret_cast<const u32x2*>(ws_o + slot * D + d0));
  }
  return acc;
}

__device__ __forceinline__ u32x2 pack_bf16x4(const f32x4& acc, float inv) {
  u32x2 w2;
  w2[0] = static_cast<uint32_t>(f32_to_bf16(acc[0] * inv)) |
          (static_cast<uint32_t>(f32_to_bf16(acc[1] * inv)) << 16);
  w2[1] = static_cast<uint32_t>(f32_to_bf16(acc[2] * inv)) |
          (static_cast<uint32_t>(f32_to_bf16(acc[3] * inv)) << 16);
  return w2;
}

// One work-group's share of a prefill launch: item x of slice c, where
// x = kvh + H_kv (hg + n_head_groups (split + n_split pt')) and the
// position tile is pt = n_pos_tiles - 1 - pt' (longest rows first).  smem:
// 4 * stage_bytes<D>() bytes of LDS.
//
// kVarlen (the fused decode + prefill launch): `start_pos` holds each
// slice's context length after the slice (its start is that minus the
// slice length), the rows of cu_q_lens count from cu_q_lens[0] rather than
// zero, and when the key range is split the last of a group's work-groups
// to finish merges the group's partials (merge_counters: one per group,
// zero before and after).
template <typename CacheT, int D, bool kVarlen, int BS>
__device__ __attribute__((always_inline)) inline void prefill_block(
    uint8_t* __restrict__ smem, int x, const int c,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ start_pos,
    const typename CacheT::raw* __restrict__ k_cache,
    const typename CacheT::raw* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    int32_t max_blocks, int32_t num_blocks, int32_t H_q, PfGeom geo, float score_scale,
    float v_scale, float* __restrict__ ws_ml, uint16_t* __restrict__ ws_o, int32_t ws_rows,
    int32_t* __restrict__ merge_counters) {
  constexpr int NKS = D / 16;  // 16-dim MFMA steps of Q K^T
  constexpr int NDT = D / 32;  // 32-dim tiles of O^T
  using Loader = TileLoader<CacheT, D, BS>;
  constexpr int NLD = Loader::NLD;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 5;   // which half of the wave (MFMA k-group)
  const int col = lane & 31; // the lane's query within the wave

  const int kvh = x % geo.H_kv;
  x /= geo.H_kv;
  const int hg = x % geo.n_head_groups;
  x /= geo.n_head_groups;
  const int split = x % geo.n_split;
  const int pt = geo.n_pos_tiles - 1 - x / geo.n_split;  // longest rows first

  const int32_t q0 = cu_q_lens[c];
  const int32_t qlen = cu_q_lens[c + 1] - q0;
  // (a context shorter than its slice is invalid; clamped so that no table
  // index goes negative)
  const int32_t P0 = kVarlen ? max(start_pos[c] - qlen, 0) : start_pos[c];
  const int32_t rbase = kVarlen ? cu_q_lens[0] : 0;  // row of the launch's first query
  const int pos_per_group = kPfRows * geo.psub;
  const int grp0 = pt * pos_per_group;
  if (grp0 >= qlen) return;
  const int grp_end = min(grp0 + pos_per_group, qlen);
  const int32_t kv_end = P0 + grp_end;  // keys this group needs: [0, kv_end)

  const int n_tiles = (kv_end + kPfKeys - 1) / kPfKeys;
  const int per = (n_tiles + geo.n_split - 1) / geo.n_split;
  const int t0 = split * per;
  const int t1 = min(n_tiles, t0 + per);

  // this wave's query head and positions
  const int hi = wave % geo.hpw, ps = wave / geo.hpw;
  const int hq_in_group = hg * kPfWaves + hi;
  const bool active = ps < geo.psub && hq_in_group < geo.G;
  const int head = kvh * geo.G + hq_in_group;
  const int w0 = grp0 + ps * kPfRows;  // first position (relative to the slice)
  const bool wave_live = active && w0 < qlen;
  const int my_rel = min(w0 + col, qlen - 1);
  const int32_t qpos = P0 + my_rel;   // absolute position (clamped for rows past the end)
  const bool row_ok = wave_live && (w0 + col) < qlen;
  const int32_t wave_first_pos = P0 + w0;

  // Q fragment: query `col`, dims 16 ks + 8 g .. + 7
  bf16x8 qf[NKS];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + my_rel) * H_q + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (row_ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    // Settle the Q loads here: otherwise the counter bookkeeping at the loop
    // head cannot tell them from the K/V prefetch and waits for all loads
    // before every tile's first MFMA.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  f32x16 o[NDT];
#pragma unroll
  for (int n = 0; n < NDT; ++n)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[n][j] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int32_t* table = block_tables + static_cast<int64_t>(c) * max_blocks;
  const int32_t n_blk = min((kv_end + BS - 1) / BS, max_blocks);
  // A tile's block ids are fetched by a vector load one iteration before
  // its K/V loads are issued: lanes 0..n-1 take the tile's n entries
  // (entries past the context repeat the last one); each is clamped into
  // the pool where it is used.
  auto fetch_ids = [&](int t) -> int32_t {
    constexpr int n = Loader::kIdsPerTile;
    return table[min(t * n + (lane & (n - 1)), n_blk - 1)];
  };

  const Loader ld(wave, lane);
  const int v_lane = v_off(col, g);

  // Software pipeline inside each wave.  Iteration t enters with the fp16
  // weights P(t-1) and the scores S(t).  One straight run of 32 MFMAs then
  // computes S(t+1) = K(t+1) Q^T and O^T += V(t-1)^T P(t-1)^T; none of them
  // waits for the vector work of the same iteration, which in between turns
  // S(t) into P(t) against the current softmax reference.  Only when P(t)
  // would leave fp16 (checked on its row sums after the run, rare) is the
  // reference raised and P(t) formed again.  K/V tiles rotate through four
  // LDS stages: tile t is stored during iteration t-2, read as K in
  // iteration t-1 and as V in iteration t+1.
  auto stage = [&](int t) { return smem + ((t - t0) & 3) * stage_bytes<D>(); };
  constexpr int NQK = 2 * NKS;       // S MFMAs per tile
  constexpr int NPV = 4 * NDT;       // O MFMAs per tile
  constexpr int NM = NQK + NPV;
  constexpr int WPS = 32 / NM;       // weights formed per MFMA slot
  static_assert(WPS * NM == 32, "32 scores per lane and tile");
  constexpr int PD = 2;              // operand reads issued this many MFMAs ahead
  constexpr int kLd0 = NLD;          // first slot with a tile load
  constexpr int kLdEvery = 4;        // one tile load every this many MFMA slots
  static_assert(kLd0 + kLdEvery * NLD < NM, "the tile loads fit the slots");

  u32x4 regs[NLD];
  // block ids of the next tile to load (ids_a) and of the one after (ids_b):
  // fetched two loads ahead, so their latency never delays a tile load
  int32_t ids_a = fetch_ids(t0);
  int32_t ids_b = fetch_ids(min(t0 + 1, t1 - 1));
  auto load_tile = [&](int t) {  // tiles past the range reload the last one
    const int tc = min(t, t1 - 1);
    ld.load(regs, k_cache, v_cache, ids_a, kvh, geo.H_kv, num_blocks);
    ids_a = ids_b;
    ids_b = fetch_ids(min(tc + 2, t1 - 1));
  };
  auto store_tile = [&](int t) {
    ld.store(regs, stage(t), kv_end - min(t, t1 - 1) * kPfKeys);
  };
  auto zero_v_tail = [&](uint8_t* v_lds, int valid) {
    for (int idx = tid; idx < D * 8; idx += kPfThreads) {
      const int d = idx >> 3, c = idx & 7;
      if (8 * c + 7 >= valid) {
        f16x8* p = reinterpret_cast<f16x8*>(v_lds + v_off(d, c));
        f16x8 v = *p;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * c + j >= valid) v[j] = static_cast<_Float16>(0.0f);
        *p = v;
      }
    }
  };
  auto mask_scores = [&](f32x16* s, int t) {
    const int lim = qpos - t * kPfKeys - 8 * g;  // largest admissible key offset
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int off = 32 * h + 16 * (j >> 3) + (j & 7);
        s[h][j] = off <= lim ? s[h][j] : -__builtin_inff();
      }
  };
  // the score scale is positive, so maxima are taken on raw scores
  // S^T of the 64 keys of a stage
  auto qk_stage = [&](const uint8_t* k_lds, f32x16* s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[h][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            k_lds + (2 * ks + g) * (kPfKeys * 16) + (32 * h + col) * 16);
        s[h] = mfma32x32x16(a, qf[ks], s[h]);
      }
    }
  };
  auto half_max = [&](const f32x16& s) {
    // scores are never NaN: plain three-way maxima, no quieting
    float m;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(s[0]), "v"(s[1]), "v"(s[2]));
#pragma unroll
    for (int j = 3; j < 15; j += 2)
      asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(s[j]), "v"(s[j + 1]));
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(s[15]));
    return m;
  };
  // The softmax reference m_run (log2 domain) starts at the maximum of the
  // first tile and is raised only when a tile's weights would leave fp16:
  // a lane whose 32 weights of a tile sum beyond kPfSafe (or overflow).
  // Any reference gives the same normalised result; this one never lies
  // above the running maximum, so the largest weight seen so far is >= 1.
  float mu = 0.f;                    // reference the exponentials use
  // lane maximum of raw scores -> the query's maximum, scaled
  auto query_max = [&](const f32x16* s) {
    const float mx = fmaxf(half_max(s[0]), half_max(s[1]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * score_scale;
  };
  // raise the reference to m_new (>= m_run), rescaling l and O^T
  auto raise_to = [&](float m_new) {
    const float alpha =
        m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[n][j] *= alpha;
    m_run = m_new;
    mu = m_run == -__builtin_inff() ? 0.f : m_run;
  };
  // fp16 weights of S (32 per lane) against mu, and their sum
  auto weights = [&](const f32x16* s, f16x8* p) {
    const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      const int u = e >> 3, i8 = e & 7;
      const f16x2 h2 = {static_cast<_Float16>(__builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[u >> 1][8 * (u & 1) + i8], score_scale, -mu))),
                        static_cast<_Float16>(__builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[u >> 1][8 * (u & 1) + i8 + 1], score_scale, -mu)))};
      p[u][i8] = h2[0];
      p[u][i8 + 1] = h2[1];
      sum = __builtin_amdgcn_fdot2(h2, ones, sum, false);
    }
    return sum;
  };

  // One iteration.  sc: S(t) in, sn: S(t+1) out, pp: P(t-1) in, pn: P(t) out.
  auto body = [&](auto masked_next, int t, f32x16* sc, f32x16* sn, const f16x8* pp, f16x8* pn) {
    // Tile t+2 (loaded during the last iteration) goes into its stage in the
    // first slots; the global loads of tile t+3 follow, spread over the
    // slots so that the waves do not queue for the address unit at once,
    // and have a whole iteration to arrive.
    const int t_ld = min(t + 3, t1 - 1);
    uint8_t* st_lds = stage(t + 2);
    const uint8_t* k_lds = stage(t + 1);
    const uint8_t* v_lds = stage(t - 1) + D * kPfKeys * 2;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j) sn[h][j] = 0.f;
    // MFMA slot i < NQK: S step i (h = i & 1, ks = i >> 1); slot NQK + j: O
    // step j (u = j / NDT, n = j % NDT)
    auto operand = [&](int i) -> u32x4 {
      if (i < NQK)
        return *reinterpret_cast<const u32x4*>(k_lds + (2 * (i >> 1) + g) * (kPfKeys * 16) +
                                                (32 * (i & 1) + col) * 16);
      const int j = i - NQK;
      return *reinterpret_cast<const u32x4*>(v_lds + v_lane + (j % NDT) * 4096 + (j / NDT) * 512);
    };
    u32x4 opnd[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) opnd[i] = operand(i);
    const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    float l_tile = 0.f;
    float w_even = 0.f;  // first weight of a pair whose second is still to come
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + PD < NM) opnd[(i + PD) % (PD + 1)] = operand(i + PD);
      if (i < NLD) ld.store1(regs[i], i, st_lds);
      if (i >= kLd0 && (i - kLd0) % kLdEvery == 0 && (i - kLd0) / kLdEvery < NLD)
        ld.load1(regs[(i - kLd0) / kLdEvery], (i - kLd0) / kLdEvery, k_cache, v_cache, ids_a,
                 kvh, geo.H_kv, num_blocks);
      if (i == kLd0 + kLdEvery * NLD) {
        ids_a = ids_b;
        ids_b = fetch_ids(min(t_ld + 2, t1 - 1));
      }
      if (i < NQK) {
        sn[i & 1] = mfma32x32x16(__builtin_bit_cast(bf16x8, opnd[i % (PD + 1)]), qf[i >> 1],
                                 sn[i & 1]);
      } else {
        const int j = i - NQK;
        o[j % NDT] = mfma32x32x16(__builtin_bit_cast(f16x8, opnd[i % (PD + 1)]), pp[j / NDT],
                                  o[j % NDT]);
        // S(t+1) is complete two slots after its last MFMA: mask it where
        // it reaches the diagonal
        if constexpr (decltype(masked_next)::value)
          if (j == 1) mask_scores(sn, t + 1);
      }
      // weights of S(t) spread evenly over all the slots: slot i forms
      // e = WPS i .. WPS i + WPS - 1 (e = 8 u + i8: key 16 u + i8 of the
      // lane's half); a pair goes to fp16 and into the row sum once its
      // second weight exists.  Each value is pinned to its slot (empty asm),
      // not left to sink to where it is next used.
#pragma unroll
      for (int q2 = 0; q2 < WPS; ++q2) {
        const int e = WPS * i + q2;
        const int u = e >> 3, i8 = e & 7;
        float w = __builtin_amdgcn_exp2f(
            __builtin_fmaf(sc[u >> 1][8 * (u & 1) + i8], score_scale, -mu));
        if (e & 1) {
          f16x2 h2 = {static_cast<_Float16>(w_even), static_cast<_Float16>(w)};
          asm volatile("" : "+v"(h2));
          pn[u][i8 - 1] = h2[0];
          pn[u][i8] = h2[1];
          l_tile = __builtin_amdgcn_fdot2(h2, ones, l_tile, false);
          asm volatile("" : "+v"(l_tile));
        } else {
          asm volatile("" : "+v"(w));
          w_even = w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P(t) left fp16 (rare: S(t) far above the reference): recompute S(t)
    // from tile t's K, still in its stage, raise the reference to its
    // maximum (O^T holds P(t-1) V(t-1) by now) and form P(t) again
    if (__builtin_amdgcn_ballot_w64(!(l_tile <= kPfSafe)) != 0) {
      qk_stage(stage(t), sc);
      if (t * kPfKeys + kPfKeys - 1 > wave_first_pos) mask_scores(sc, t);
      raise_to(fmaxf(m_run, query_max(sc)));
      l_tile = weights(sc, pn);
    }
    l_run += l_tile;
    // V of keys past the context must be zero, not stale cache bits.  The
    // tail is cleared in tile t+1, whose pieces every wave stored during
    // the last iteration (complete at its closing barrier) and whose V is
    // first read in iteration t+2; this iteration reads only its K.  (The
    // tile stored in this iteration cannot be cleared here: a wave still
    // storing a piece would race the read-modify-write of another.)
    const int valid_nx = kv_end - min(t + 1, t1 - 1) * kPfKeys;
    if (valid_nx < kPfKeys) zero_v_tail(stage(t + 1) + D * kPfKeys * 2, valid_nx);
    __syncthreads();
  };

  if (t0 < t1) {
    load_tile(t0);
    store_tile(t0);
    load_tile(t0 + 1);
    store_tile(t0 + 1);
    load_tile(t0 + 2);  // stored by iteration t0
    {
      // iteration t0 multiplies zero weights by the V half of the stage
      // before it: clear that half so that no stale bits become NaN
      uint8_t* vz = stage(t0 - 1) + D * kPfKeys * 2;
      for (int i = tid; i < D * kPfKeys * 2 / 16; i += kPfThreads)
        *reinterpret_cast<u32x4*>(vz + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    f32x16 sA[2], sB[2];
    f16x8 pA[4], pB[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) pA[u][i] = static_cast<_Float16>(0.0f);
    // S(t0) and the first reference, its maximum
    qk_stage(stage(t0), sA);
    if (t0 * kPfKeys + kPfKeys - 1 > wave_first_pos) mask_scores(sA, t0);
    m_run = query_max(sA);
    mu = m_run == -__builtin_inff() ? 0.f : m_run;
    // iteration t masks S(t+1) when tile t+1 reaches past the wave's first
    // position, i.e. from tile t_mask on
    const int t_mask = (wave_first_pos + 1) / kPfKeys;
    int t = t0;
    for (; t + 2 < min(t_mask, t1); t += 2) {
      body(std::false_type{}, t, sA, sB, pA, pB);
      body(std::false_type{}, t + 1, sB, sA, pB, pA);
    }
    for (; t + 1 < t1; t += 2) {
      body(std::true_type{}, t, sA, sB, pA, pB);
      body(std::true_type{}, t + 1, sB, sA, pB, pA);
    }
    const f16x8* p_last = pA;
    int t_last = t - 1;
    if (t < t1) {
      body(std::true_type{}, t, sA, sB, pA, pB);
      p_last = pB;
      t_last = t;
    }
    // O^T += V(last)^T P(last)^T; every owed rescale is already applied
    const uint8_t* v_lds = stage(t_last) + D * kPfKeys * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(v_lds + v_lane + n * 4096 + u * 512);
        o[n] = mfma32x32x16(a, p_last[u], o[n]);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const int64_t row = q0 + w0 + col;
  if (geo.n_split == 1) {
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? v_scale / l_tot : 0.f;
    uint16_t* orow = out + (row * H_q + head) * D;
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = 32 * n + 8 * jq + 4 * g;
        u32x2 w;
        w[0] = static_cast<uint32_t>(f32_to_bf16(o[n][4 * jq] * inv)) |
               (static_cast<uint32_t>(f32_to_bf16(o[n][4 * jq + 1] * inv)) << 16);
        w[1] = static_cast<uint32_t>(f32_to_bf16(o[n][4 * jq + 2] * inv)) |
               (static_cast<uint32_t>(f32_to_bf16(o[n][4 * jq + 3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    return;
  }
  // split key range: this work-group's partial softmax state
  const int64_t wrow = row - rbase;   // row inside the workspace
  const bool ws_ok = row_ok && wrow < ws_rows;
  // (the output normalised by this split's own weight sum, as fp16)
  if (ws_ok) {
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t slot = (static_cast<int64_t>(split) * ws_rows + wrow) * H_q + head;
    uint16_t* po = ws_o + slot * D;
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = 32 * n + 8 * jq + 4 * g;
        *reinterpret_cast<u32x2*>(po + d) = pf_pack_f16x4(
            f32x4{o[n][4 * jq], o[n][4 * jq + 1], o[n][4 * jq + 2], o[n][4 * jq + 3]} * inv_l);
      }
    if (g == 0) {
      ws_ml[2 * slot] = m_run;
      ws_ml[2 * slot + 1] = l_tot;
    }
  }
  if constexpr (kVarlen) {
    // The last of the group's n_split work-groups merges its partials.
    // Publication: every wave's partial stores, then the barrier, then one
    // agent-scope release (the counter bump by thread 0: one write-back of
    // the L2's dirty lines per work-group, nothing invalidated, so the other
    // work-groups' K/V tiles stay cached).  The work-group that completes
    // the count acquires at agent scope (thread 0, before the barrier that
    // releases its waves to read the partials) and clears the counter.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();  // all waves are past the stages: word 0 is free
    int32_t* flag = reinterpret_cast<int32_t*>(smem);
    if (tid == 0) {
      const int64_t gi =
          ((static_cast<int64_t>(c) * geo.n_pos_tiles + pt) * geo.n_head_groups + hg) * geo.H_kv +
          kvh;
      const int32_t prev = __hip_atomic_fetch_add(&merge_counters[gi], 1, __ATOMIC_RELEASE,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const int32_t last = prev == geo.n_split - 1;
      if (last) {
        __hip_atomic_store(&merge_counters[gi], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      *flag = last;
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (!last || !ws_ok) return;
    // The merge of the pf_merge_* helpers (same operations in the same
    // order, so the same bits as the merge kernel), arranged for latency:
    // each split's pieces (this work-group's own as it stored them) are
    // loaded together.
    const int64_t stride = static_cast<int64_t>(ws_rows) * H_q;
    const int64_t pair = wrow * H_q + head;
    // (m, l) of every split, loaded without branches so that the loads are
    // in flight together (splits past n_split reread the last one and are
    // then ignored)
    float mj[kPfMaxSplit], lj[kPfMaxSplit];
#pragma unroll
    for (int j = 0; j < kPfMaxSplit; ++j) {
      const int jj = min(j, geo.n_split - 1);
      const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * (jj * stride + pair));
      mj[j] = ml.x;
      lj[j] = j >= geo.n_split ? 0.f : ml.y;
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kPfMaxSplit; ++j)
      if (j < geo.n_split && lj[j] > 0.f) M = fmaxf(M, mj[j]);
    float L = 0.f;
#pragma unroll
    for (int j = 0; j < kPfMaxSplit; ++j)
      if (j < geo.n_split && lj[j] > 0.f) L += pf_merge_weight(mj[j], lj[j], M);
    const float inv = L > 0.f ? v_scale / L : 0.f;
    f32x4 acc[NDT][4];
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) acc[n][jq] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < geo.n_split; ++j) {
      if (!(lj[j] > 0.f)) continue;
      const float w = pf_merge_weight(mj[j], lj[j], M);
      const uint16_t* po = ws_o + (j * stride + pair) * D;
      u32x2 v[NDT][4];
#pragma unroll
      for (int n = 0; n < NDT; ++n)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq)
          v[n][jq] = *reinterpret_cast<const u32x2*>(po + 32 * n + 8 * jq + 4 * g);
#pragma unroll
      for (int n = 0; n < NDT; ++n)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) acc[n][jq] += w * pf_unpack_f16x4(v[n][jq]);
    }
    uint16_t* orow = out + (row * H_q + head) * D;
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<u32x2*>(orow + 32 * n + 8 * jq + 4 * g) = pack_bf16x4(acc[n][jq], inv);
  }
}

}  // namespace
}  // namespace pa
