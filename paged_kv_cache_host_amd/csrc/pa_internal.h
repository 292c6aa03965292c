// Declarations shared by the host translation units of libpa.
#pragma once

#include "pa.h"

#include <hip/hip_runtime.h>

namespace pa {

// Kernels whose launches the optional timing facility can record.
enum KernelId {
  kCacheWrite = 0,
  kDecode,
  kDecodeMerge,
  kPrefill,
  kPrefillMerge,
  kGeneric,
  kKernelCount
};

// Record a HIP event before (begin) or after (!begin) a kernel launch on
// `st` when timing is enabled (pa_timing_enable); a no-op otherwise.
void timing_mark(hipStream_t st, KernelId k, bool begin);

// Record a printf-style message as the calling thread's last error and
// return `st`.
pa_status fail(pa_status st, const char* fmt, ...);

}  // namespace pa
