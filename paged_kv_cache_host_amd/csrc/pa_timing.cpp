// Optional per-kernel timing of libpa's own launches.
//
// For the kernels selected by a bit mask, each launch carries a pair of HIP
// events attached to the launch itself (hipExtLaunchKernel), which take the
// kernel's start and end times; pa_timing_query waits for them and reports
// how many launches of a kernel were kept and their mean and total
// duration; a period n times only every n-th launch of a kernel.  Disabled
// (the default), the hook costs one flag test per launch.  The events are not free: the start event is one more command in
// the stream, and a kernel whose end is observable from the host makes the
// device write its dirty cache lines back when it ends (a few microseconds
// each, measured on MI355X), so only the kernels of interest should be
// selected.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCapacity = 4096;  // launches kept per kernel between resets
constexpr int kReserve = 64;     // event pairs created when a kernel is selected

struct Slot {
  hipEvent_t start = nullptr, stop = nullptr;
};

struct Track {
  std::vector<Slot> slots;  // events are created on first use and reused
  int count = 0;            // launches timed since the last reset
  int64_t seen = 0;         // launches since the last reset
};

std::mutex g_mu;
std::atomic<int32_t> g_mask{0};  // bit k: time kernel k
int32_t g_every = 1;             // time launches 0, every, 2 * every, ... of a kernel
Track g_tracks[kKernelCount];

const char* kNames[kKernelCount] = {"cache_write",   "decode",  "decode_merge",
                                    "prefill",       "prefill_merge", "generic",
                                    "stage",         "stage_cache_write", "varlen",
                                    "decode_step"};

}  // namespace

void timing_events(KernelId k, hipStream_t, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!(g_mask.load(std::memory_order_relaxed) & (1 << k))) return;
  std::lock_guard<std::mutex> lock(g_mu);
  Track& t = g_tracks[k];
  if (t.seen++ % g_every != 0 || t.count >= kCapacity) return;
  if (static_cast<int>(t.slots.size()) <= t.count) {
    Slot s;
    if (hipEventCreate(&s.start) != hipSuccess || hipEventCreate(&s.stop) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    t.slots.push_back(s);
  }
  *start = t.slots[t.count].start;
  *stop = t.slots[t.count].stop;
  ++t.count;
}

void timing_rollback(KernelId k, hipStream_t, hipEvent_t stop) {
  // the launch failed, so its events were never recorded: forget them
  std::lock_guard<std::mutex> lock(g_mu);
  Track& t = g_tracks[k];
  if (t.count > 0 && t.slots[t.count - 1].stop == stop) --t.count;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_timing_enable(int32_t mask, int32_t every) {
  if (every < 1) return fail(PA_ERR_INVALID, "pa_timing_enable: every=%d must be >= 1", every);
  std::lock_guard<std::mutex> lock(g_mu);
  g_mask = mask;
  g_every = every;
  for (int k = 0; k < kKernelCount; ++k) {
    Track& t = g_tracks[k];
    t.count = 0;
    t.seen = 0;
    // the events of a selected kernel's first launches are created here,
    // not inside the launches (and a timed region) that use them
    if (mask & (1 << k)) {
      while (static_cast<int>(t.slots.size()) < kReserve) {
        Slot sl;
        if (hipEventCreate(&sl.start) != hipSuccess) break;
        if (hipEventCreate(&sl.stop) != hipSuccess) {
          (void)hipEventDestroy(sl.start);
          break;
        }
        t.slots.push_back(sl);
      }
      (void)hipGetLastError();
    }
  }
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
