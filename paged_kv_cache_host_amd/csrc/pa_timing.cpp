// Optional per-kernel timing of libpa's own launches.
//
// For the kernels selected by a bit mask, the launchers record a HIP event
// before and after each launch on the caller's stream; pa_timing_query waits
// for the recorded events and reports how many launches of a kernel were
// recorded and their mean and total duration.  Disabled (the default), the
// hooks cost one flag test per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCapacity = 4096;  // launches recorded per kernel between resets

struct Slot {
  hipEvent_t start = nullptr, stop = nullptr;
};

struct Track {
  std::vector<Slot> slots;  // events are created on first use and reused
  int count = 0;
};

std::mutex g_mu;
std::atomic<int32_t> g_mask{0};  // bit k: record kernel k
Track g_tracks[kKernelCount];

const char* kNames[kKernelCount] = {"cache_write", "decode",        "decode_merge",
                                    "prefill",     "prefill_merge", "generic"};

}  // namespace

void timing_mark(hipStream_t st, KernelId k, bool begin) {
  if (!(g_mask.load(std::memory_order_relaxed) & (1 << k))) return;
  std::lock_guard<std::mutex> lock(g_mu);
  Track& t = g_tracks[k];
  if (begin) {
    if (t.count >= kCapacity) return;
    if (static_cast<int>(t.slots.size()) <= t.count) {
      Slot s;
      if (hipEventCreate(&s.start) != hipSuccess || hipEventCreate(&s.stop) != hipSuccess) {
        (void)hipGetLastError();
        return;
      }
      t.slots.push_back(s);
    }
    (void)hipEventRecord(t.slots[t.count].start, st);
  } else {
    if (t.count >= kCapacity || static_cast<int>(t.slots.size()) <= t.count) return;
    (void)hipEventRecord(t.slots[t.count].stop, st);
    ++t.count;
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_timing_enable(int32_t mask) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_mask = mask;
  for (auto& t : g_tracks) t.count = 0;
  return PA_OK;
}

extern "C" pa_status pa_timing_query(const char* kernel, int32_t* count, float* mean_us,
                                     float* total_us) {
  if (!kernel || !count || !mean_us || !total_us)
    return fail(PA_ERR_INVALID, "pa_timing_query: NULL argument");
  int k = -1;
  for (int i = 0; i < kKernelCount; ++i)
    if (std::strcmp(kernel, kNames[i]) == 0) k = i;
  if (k < 0) return fail(PA_ERR_INVALID, "pa_timing_query: unknown kernel name '%s'", kernel);
  std::lock_guard<std::mutex> lock(g_mu);
  const Track& t = g_tracks[k];
  double total_ms = 0.0;
  for (int i = 0; i < t.count; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(t.slots[i].stop) != hipSuccess ||
        hipEventElapsedTime(&ms, t.slots[i].start, t.slots[i].stop) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_DEVICE, "pa_timing_query: event timing failed");
    }
    total_ms += ms;
  }
  *count = t.count;
  *total_us = static_cast<float>(total_ms * 1e3);
  *mean_us = t.count ? static_cast<float>(total_ms * 1e3 / t.count) : 0.f;
  return PA_OK;
}
