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
#include "pa_copy.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// grid: stage_groups(n); block: 256.  n: words of type W (8 bytes when both
// addresses and the size allow it, else 4).
template <typename W>
__global__ __launch_bounds__(kStageThreads) void stage_kernel(W* __restrict__ dst,
                                                              const W* __restrict__ src,
                                                              int64_t n) {
  stage_words<W>(dst, src, n, blockIdx.x, gridDim.x);
}

template <typename W>
pa_status launch_stage(hipStream_t st, void* dst, const void* src_dev, size_t bytes) {
  const int64_t n = static_cast<int64_t>(bytes / sizeof(W));
  const int grid = stage_groups(n);
  const hipError_t e = launch(kStage, stage_kernel<W>, dim3(grid), dim3(kStageThreads), 0, st,
                              static_cast<W*>(dst), static_cast<const W*>(src_dev), n);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "pa_stage: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

pa_status pinned_alias(const char* who, const void* src_host, void** src_dev) {
  *src_dev = nullptr;
  if (!src_host) return fail(PA_ERR_INVALID, "%s: NULL source", who);
  void* p = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&p, const_cast<void*>(src_host), 0);
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID, "%s: source is not pinned host memory (%s)", who,
                hipGetErrorString(e));
  }
  *src_dev = p;
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_pinned_alias(const void* src_host, void** src_dev) {
  if (!src_dev) return fail(PA_ERR_INVALID, "pa_pinned_alias: NULL result pointer");
  return pinned_alias("pa_pinned_alias", src_host, src_dev);
}

extern "C" pa_status pa_stage(void* stream, void* dst, const void* src_host, size_t bytes) {
  if (bytes == 0) return PA_OK;
  if (!dst || !src_host) return fail(PA_ERR_INVALID, "pa_stage: NULL buffer");
  if (bytes % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(src_host) % 4 != 0)
    return fail(PA_ERR_INVALID, "pa_stage: bytes=%zu and both addresses must be multiples of 4",
                bytes);
  void* src_dev = nullptr;
  const pa_status ps = pinned_alias("pa_stage", src_host, &src_dev);
  if (ps != PA_OK) return ps;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (bytes % 8 == 0 && reinterpret_cast<uintptr_t>(dst) % 8 == 0 &&
      reinterpret_cast<uintptr_t>(src_dev) % 8 == 0)
    return launch_stage<uint64_t>(st, dst, src_dev, bytes);
  return launch_stage<uint32_t>(st, dst, src_dev, bytes);
}
