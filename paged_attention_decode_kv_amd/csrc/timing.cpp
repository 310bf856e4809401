// Event-pair timing of the library's kernel phases (pkv_timing_enable / _read).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"

namespace pkv {
namespace {

constexpr int kPhases = 6;

struct PhaseLog {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;  // recorded, not yet read
  std::vector<hipEvent_t> spare;                           // reusable events
  hipEvent_t open = nullptr;                               // start of the current launch
  double total_ms = 0.0;
  int64_t launches = 0;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
PhaseLog g_log[kPhases];

hipEvent_t take(PhaseLog& p) {
  if (!p.spare.empty()) {
    hipEvent_t e = p.spare.back();
    p.spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Returns an event to the phase's spares; if that cannot grow, the event is destroyed
// (these run inside C-ABI calls, which no exception may leave).
void keep_spare(PhaseLog& p, hipEvent_t e) noexcept {
  try {
    p.spare.push_back(e);
  } catch (...) {
    (void)hipEventDestroy(e);
  }
}

}  // namespace

void timing_enable(bool on) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_on = on;
}

// A stream under capture records nodes, not work: events there would never complete
// on their own, so captured launches go untimed.
static bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

void timing_begin(int phase, hipStream_t stream) {
  if (!g_on || capturing(stream)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  PhaseLog& p = g_log[phase];
  p.open = take(p);
  if (p.open && hipEventRecord(p.open, stream) != hipSuccess) p.open = nullptr;
}

void timing_end(int phase, hipStream_t stream) {
  if (!g_on || capturing(stream)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  PhaseLog& p = g_log[phase];
  if (!p.open) return;
  hipEvent_t stop = take(p);
  if (!stop) return;
  if (hipEventRecord(stop, stream) != hipSuccess) {
    keep_spare(p, p.open);
    keep_spare(p, stop);
    p.open = nullptr;
    return;
  }
  try {
    p.pending.emplace_back(p.open, stop);
  } catch (...) {   // the sample is dropped
    keep_spare(p, p.open);
    keep_spare(p, stop);
  }
  p.open = nullptr;
}

hipError_t timing_read(int phase, double* total_ms, int64_t* launches, bool reset) {
  std::lock_guard<std::mutex> lock(g_mu);
  PhaseLog& p = g_log[phase];
  size_t done = 0;
  for (; done < p.pending.size(); ++done) {
    const auto& pr = p.pending[done];
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {   // the samples already summed leave the list
      p.pending.erase(p.pending.begin(), p.pending.begin() + done);
      return e;
    }
    p.total_ms += ms;
    p.launches += 1;
    keep_spare(p, pr.first);
    keep_spare(p, pr.second);
  }
  p.pending.clear();
  *total_ms = p.total_ms;
  *launches = p.launches;
  if (reset) {
    p.total_ms = 0.0;
    p.launches = 0;
  }
  return hipSuccess;
}

namespace {
std::atomic<int> g_chunk_min{kDefaultChunkMin};
std::atomic<int> g_chunk_max{kDefaultChunkMax};
std::atomic<int> g_decode_waves{kDefaultDecodeWaves};
std::atomic<int> g_items_per_group{kDefaultItemsPerGroup};
std::atomic<int> g_deal_static{kDefaultDealStatic};
std::atomic<int> g_lds_stage{kDefaultLdsStage};
std::atomic<int> g_max_query_group{kDefaultMaxQueryGroup};
std::atomic<int> g_mfma{kDefaultMfma};
std::atomic<int> g_groups_per_cu{kDefaultGroupsPerCu};
std::atomic<int> g_solo_tokens{kDefaultSoloTokens};

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }
}  // namespace

int tuning_chunk_min() { return g_chunk_min.load(std::memory_order_relaxed); }
int tuning_chunk_max() { return g_chunk_max.load(std::memory_order_relaxed); }
int tuning_decode_waves() { return g_decode_waves.load(std::memory_order_relaxed); }
int tuning_items_per_group() { return g_items_per_group.load(std::memory_order_relaxed); }
int tuning_deal_static() { return g_deal_static.load(std::memory_order_relaxed); }
int tuning_lds_stage() { return g_lds_stage.load(std::memory_order_relaxed); }
int tuning_max_query_group() { return g_max_query_group.load(std::memory_order_relaxed); }
int tuning_mfma() { return g_mfma.load(std::memory_order_relaxed); }
int tuning_groups_per_cu() { return g_groups_per_cu.load(std::memory_order_relaxed); }
int tuning_solo_tokens() { return g_solo_tokens.load(std::memory_order_relaxed); }

bool set_tuning(int chunk_min, int chunk_max, int decode_waves, int items_per_group,
                int deal, int staging, int max_query_group, int mfma, int groups_per_cu,
                int solo_tokens) {
  const int lo = chunk_min ? chunk_min : tuning_chunk_min();
  const int hi = chunk_max ? chunk_max : tuning_chunk_max();
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
  g_chunk_min.store(lo);
  g_chunk_max.store(hi);
  if (decode_waves != 0) g_decode_waves.store(decode_waves);
  if (items_per_group != 0) g_items_per_group.store(items_per_group);
  if (deal != 0) g_deal_static.store(deal == 1 ? 1 : 0);
  if (staging != 0) g_lds_stage.store(staging == 2 ? 1 : 0);
  if (max_query_group != 0) g_max_query_group.store(max_query_group);
  if (mfma != 0) g_mfma.store(mfma == 1 ? 1 : 0);
  if (groups_per_cu != 0) g_groups_per_cu.store(groups_per_cu);
  if (solo_tokens != 0) g_solo_tokens.store(solo_tokens);
  return true;
}

}  // namespace pkv
