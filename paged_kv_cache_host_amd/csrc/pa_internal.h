// Declarations shared by the host translation units of libpa.
#pragma once

#include "pa.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace pa {

// Kernels whose launches the optional timing facility can record.
enum KernelId {
  kCacheWrite = 0,
  kDecode,
  kDecodeMerge,
  kPrefill,
  kPrefillMerge,
  kGeneric,
  kStage,
  kStageCacheWrite,
  kVarlen,
  kDecodeStep,
  kKernelCount
};

// The (start, stop) events for the next launch of kernel k when its timing
// is enabled (pa_timing_enable) and its record is not full; both null
// otherwise.
void timing_events(KernelId k, hipStream_t st, hipEvent_t* start, hipEvent_t* stop);

// Forget the events of a launch that failed.
void timing_rollback(KernelId k, hipStream_t st, hipEvent_t stop);

template <typename T, size_t... I>
inline hipError_t launch_packed(KernelId k, const void* fn, dim3 grid, dim3 block,
                                uint32_t shmem, hipStream_t st, T& vals,
                                std::index_sequence<I...>) {
  void* argv[] = {static_cast<void*>(&std::get<I>(vals))...};
  hipEvent_t a = nullptr, b = nullptr;
  timing_events(k, st, &a, &b);
  const hipError_t e = b ? hipExtLaunchKernel(fn, grid, block, argv, shmem, st, a, b, 0)
                         : hipLaunchKernel(fn, grid, block, argv, shmem, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    if (b) timing_rollback(k, st, b);
  }
  return e;
}

// Launch `kernel` (id k) on `st` with `args` converted to its parameter
// types.  When k is being timed, the launch itself carries its start and
// stop events (hipExtLaunchKernel), which time the kernel alone rather than
// the interval between two event records around it.
template <typename... P, typename... A>
inline hipError_t launch(KernelId k, void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem,
                         hipStream_t st, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> vals{static_cast<P>(args)...};
  return launch_packed(k, reinterpret_cast<const void*>(kernel), grid, block, shmem, st, vals,
                       std::index_sequence_for<P...>{});
}

// pa_pinned_alias with the caller's name in the error text.
pa_status pinned_alias(const char* who, const void* src_host, void** src_dev);

// Record a printf-style message as the calling thread's last error and
// return `st`.
pa_status fail(pa_status st, const char* fmt, ...);

}  // namespace pa
