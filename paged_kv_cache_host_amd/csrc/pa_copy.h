// Device bodies shared by the metadata staging kernel (pa_stage) and the
// fused staging + cache-write kernel (pa_stage_cache_write).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace pa {

constexpr int kStageThreads = 256;  // threads per work-group
constexpr int kStageUnroll = 4;     // words in flight per thread

// Work-groups that copy n words (at most 256; each thread moves 4 words per
// round, rounds stride over the groups).
inline int stage_groups(int64_t n) {
  const int64_t per_group = int64_t{kStageThreads} * kStageUnroll;
  return static_cast<int>(std::min<int64_t>((n + per_group - 1) / per_group, 256));
}

// Work-group `group` of `groups` copies its share of n words from src
// (pinned host memory, read with system-scope loads so that host writes made
// before the launch are seen whether or not the allocation is fine-grained)
// to dst (device memory).
template <typename W>
__device__ __forceinline__ void stage_words(W* __restrict__ dst, const W* __restrict__ src,
                                            int64_t n, int group, int groups) {
  const int64_t stride = static_cast<int64_t>(groups) * kStageThreads;
  for (int64_t base = static_cast<int64_t>(group) * kStageThreads + threadIdx.x; base < n;
       base += stride * kStageUnroll) {
    W v[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t i = base + u * stride;
      v[u] = i < n ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : W{0};
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < n) dst[i] = v[u];
    }
  }
}

}  // namespace pa
