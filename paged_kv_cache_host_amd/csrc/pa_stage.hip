// pa_stage: move one iteration's host-built metadata (slots, context
// lengths, block tables) from pinned host memory into a device buffer with a
// kernel on the caller's stream.
//
// LESSON "vLLM Serving Internals", "Continuous batching at the iteration
// level": the scheduler rebuilds the batch on the host every iteration, and
// the attention kernels of that iteration read the block tables it packed
// (ARTICLE 2.3: the kernel takes the per-sequence block tables and context
// lengths as inputs).  A copy-engine transfer between the kernels of one
// stream costs two cross-engine waits per iteration; a kernel in the same
// queue costs one dispatch.
//
// The source is read with system-scope loads, which stay coherent with host
// writes made before the launch whether or not the pinned allocation is
// fine-grained.
#include "pa_device.h"
#include "pa_internal.h"

#include <algorithm>

namespace pa {

constexpr int kStageThreads = 256;
constexpr int kStageUnroll = 4;

// grid: min(ceil(n / (256 * 4)), 256); block: 256.  n: 32-bit words.
__global__ __launch_bounds__(kStageThreads) void stage_kernel(uint32_t* __restrict__ dst,
                                                              const uint32_t* __restrict__ src,
                                                              int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kStageThreads;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kStageThreads + threadIdx.x; base < n;
       base += stride * kStageUnroll) {
    uint32_t v[kStageUnroll];
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t i = base + u * stride;
      v[u] = i < n ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < n) dst[i] = v[u];
    }
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_stage(void* stream, void* dst, const void* src_host, size_t bytes) {
  if (bytes == 0) return PA_OK;
  if (!dst || !src_host) return fail(PA_ERR_INVALID, "pa_stage: NULL buffer");
  if (bytes % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(src_host) % 4 != 0)
    return fail(PA_ERR_INVALID, "pa_stage: bytes=%zu and both addresses must be multiples of 4",
                bytes);
  void* src_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&src_dev, const_cast<void*>(src_host), 0);
  if (e != hipSuccess || !src_dev) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID, "pa_stage: source is not pinned host memory (%s)",
                hipGetErrorString(e));
  }
  const int64_t n = static_cast<int64_t>(bytes / 4);
  const int64_t per_group = int64_t{kStageThreads} * kStageUnroll;
  const int grid = static_cast<int>(std::min<int64_t>((n + per_group - 1) / per_group, 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  e = launch(kStage, stage_kernel, dim3(grid), dim3(kStageThreads), 0, st,
             static_cast<uint32_t*>(dst), static_cast<const uint32_t*>(src_dev), n);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_stage: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
