// Event-pair timing of the library's kernel phases (pkv_timing_enable / _read), and the
// process-wide work-split settings (pkv_set_tuning / pkv_get_tuning).
#include <hip/hip_runtime.h>

#include <atomic>
#include <thread>
#include <utility>
#include <vector>

#include "internal.h"

namespace pkv {
namespace {

// A lock whose lock() cannot throw (std::mutex::lock may throw std::system_error, and
// these functions run inside C-ABI calls that no exception may leave).
class SpinLock {
 public:
  void lock() noexcept {
    while (flag_.test_and_set(std::memory_order_acquire)) std::this_thread::yield();
  }
  void unlock() noexcept { flag_.clear(std::memory_order_release); }

 private:
  std::atomic_flag flag_ = ATOMIC_FLAG_INIT;
};

class Guard {
 public:
  explicit Guard(SpinLock& l) noexcept : l_(l) { l_.lock(); }
  ~Guard() { l_.unlock(); }
  Guard(const Guard&) = delete;
  Guard& operator=(const Guard&) = delete;

 private:
  SpinLock& l_;
};

constexpr int kPhases = 6;

struct PhaseLog {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;  // recorded, not yet read
  std::vector<hipEvent_t> spare;                           // reusable events
  // the start event of the launch in progress on each stream: a phase timed from two
  // host threads on two streams pairs each stream's start with its own stop
  std::vector<std::pair<hipStream_t, hipEvent_t>> open;
  double total_ms = 0.0;
  int64_t launches = 0;
};

SpinLock g_mu;
std::atomic<bool> g_on{false};
PhaseLog g_log[kPhases];
thread_local int g_paused = 0;   // TimingPause depth on this thread

hipEvent_t take(PhaseLog& p) noexcept {
  if (!p.spare.empty()) {
    hipEvent_t e = p.spare.back();
    p.spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Returns an event to the phase's spares; if that cannot grow, the event is destroyed.
void keep_spare(PhaseLog& p, hipEvent_t e) noexcept {
  try {
    p.spare.push_back(e);
  } catch (...) {
    (void)hipEventDestroy(e);
  }
}

// Removes and returns the open start event of `stream` (nullptr if none).
hipEvent_t take_open(PhaseLog& p, hipStream_t stream) noexcept {
  for (size_t i = 0; i < p.open.size(); ++i) {
    if (p.open[i].first == stream) {
      hipEvent_t e = p.open[i].second;
      p.open[i] = p.open.back();
      p.open.pop_back();
      return e;
    }
  }
  return nullptr;
}

}  // namespace

void timing_enable(bool on) {
  Guard lock(g_mu);
  g_on = on;
}

TimingPause::TimingPause() { ++g_paused; }
TimingPause::~TimingPause() { --g_paused; }

// A stream under capture records nodes, not work: events there would never complete
// on their own, so captured launches go untimed.
static bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

void timing_begin(int phase, hipStream_t stream) {
  if (!g_on || g_paused || capturing(stream)) return;
  Guard lock(g_mu);
  PhaseLog& p = g_log[phase];
  // a start left open on this stream (a launch that failed before its stop) is dropped
  if (hipEvent_t stale = take_open(p, stream)) keep_spare(p, stale);
  hipEvent_t e = take(p);
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    keep_spare(p, e);
    return;
  }
  try {
    p.open.emplace_back(stream, e);
  } catch (...) {   // this launch goes untimed
    keep_spare(p, e);
  }
}

void timing_end(int phase, hipStream_t stream) {
  if (!g_on || g_paused || capturing(stream)) return;
  Guard lock(g_mu);
  PhaseLog& p = g_log[phase];
  hipEvent_t start = take_open(p, stream);
  if (!start) return;
  hipEvent_t stop = take(p);
  if (!stop) {
    keep_spare(p, start);
    return;
  }
  if (hipEventRecord(stop, stream) != hipSuccess) {
    keep_spare(p, start);
    keep_spare(p, stop);
    return;
  }
  try {
    p.pending.emplace_back(start, stop);
  } catch (...) {   // the sample is dropped
    keep_spare(p, start);
    keep_spare(p, stop);
  }
}

// Sums the recorded pairs of one phase.  A pair whose events fail is dropped with its
// events destroyed, so a persistent error is reported once, not on every later read;
// the pairs summed before it stay summed.
hipError_t timing_read(int phase, double* total_ms, int64_t* launches, bool reset) {
  Guard lock(g_mu);
  PhaseLog& p = g_log[phase];
  hipError_t first_error = hipSuccess;
  for (const auto& pr : p.pending) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {
      if (first_error == hipSuccess) first_error = e;
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
      continue;
    }
    p.total_ms += ms;
    p.launches += 1;
    keep_spare(p, pr.first);
    keep_spare(p, pr.second);
  }
  p.pending.clear();
  if (first_error != hipSuccess) return first_error;
  *total_ms = p.total_ms;
  *launches = p.launches;
  if (reset) {
    p.total_ms = 0.0;
    p.launches = 0;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------------
// work-split settings
// ---------------------------------------------------------------------------------
namespace {
SpinLock g_tuning_mu;
Tuning g_tuning = {kDefaultChunkMin,      kDefaultChunkMax,   kDefaultDecodeWaves,
                   kDefaultItemsPerGroup, kDefaultDealStatic, kDefaultLdsStage,
                   kDefaultMaxQueryGroup, kDefaultMfma,       kDefaultGroupsPerCu,
                   kDefaultSoloTokens};

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }
}  // namespace

Tuning tuning_snapshot() noexcept {
  Guard lock(g_tuning_mu);
  return g_tuning;
}

bool set_tuning(int chunk_min, int chunk_max, int decode_waves, int items_per_group,
                int deal, int staging, int max_query_group, int mfma, int groups_per_cu,
                int solo_tokens) noexcept {
  Guard lock(g_tuning_mu);
  Tuning t = g_tuning;
  const int lo = chunk_min ? chunk_min : t.chunk_min;
  const int hi = chunk_max ? chunk_max : t.chunk_max;
  // validate everything before changing anything
  if (!pow2_in(lo, kMinChunkTokens, kMaxChunkTokens) ||
      !pow2_in(hi, kMinChunkTokens, kMaxChunkTokens) || lo > hi || hi / lo > kMaxChunkRatio)
    return false;
  if (decode_waves != 0 && decode_waves != 1 && decode_waves != 2 && decode_waves != 4 &&
      decode_waves != 8)
    return false;
  if (items_per_group < 0 || items_per_group > 1024) return false;
  if (deal < 0 || deal > 2) return false;
  if (staging < 0 || staging > 2) return false;
  if (max_query_group != 0 && max_query_group != 1 && max_query_group != 2 &&
      max_query_group != 4 && max_query_group != 8 && max_query_group != 16)
    return false;
  if (mfma < 0 || mfma > 2) return false;
  if (groups_per_cu < 0 || groups_per_cu > 16) return false;
  if (solo_tokens != 0 && solo_tokens != 1 &&
      !pow2_in(solo_tokens, kMinChunkTokens, kMaxSoloTokens))
    return false;
  t.chunk_min = lo;
  t.chunk_max = hi;
  if (decode_waves != 0) t.decode_waves = decode_waves;
  if (items_per_group != 0) t.items_per_group = items_per_group;
  if (deal != 0) t.deal_static = deal == 1 ? 1 : 0;
  if (staging != 0) t.lds_stage = staging == 2 ? 1 : 0;
  if (max_query_group != 0) t.max_query_group = max_query_group;
  if (mfma != 0) t.mfma = mfma == 1 ? 1 : 0;
  if (groups_per_cu != 0) t.groups_per_cu = groups_per_cu;
  if (solo_tokens != 0) t.solo_tokens = solo_tokens;
  g_tuning = t;
  return true;
}

}  // namespace pkv
