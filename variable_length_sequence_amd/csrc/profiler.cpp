// Per-kernel HIP-event timing (see profiler.h) and its C ABI.
#include "profiler.h"

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "varlen.h"

namespace vl {

namespace {

struct Rec {
  std::string name;
  hipEvent_t start = nullptr, stop = nullptr;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;        // events of the current recording
std::vector<Rec> g_free;        // reusable event pairs

void recycle_locked() {
  for (auto& r : g_recs) g_free.push_back(r);
  g_recs.clear();
}

}  // namespace

bool prof_on() { return g_on.load(std::memory_order_relaxed); }

int prof_begin(const char* kernel, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  Rec r;
  if (!g_free.empty()) {
    r = g_free.back();
    g_free.pop_back();
  } else {
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) return -1;
  }
  r.name = kernel;
  if (hipEventRecord(r.start, stream) != hipSuccess) {
    g_free.push_back(r);
    return -1;
  }
  g_recs.push_back(r);
  return int(g_recs.size()) - 1;
}

void prof_end(int slot, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (slot >= 0 && size_t(slot) < g_recs.size()) (void)hipEventRecord(g_recs[size_t(slot)].stop, stream);
}

}  // namespace vl

extern "C" {

int varlen_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(vl::g_mu);
  if (on) vl::recycle_locked();
  vl::g_on.store(on != 0);
  return VL_OK;
}

int varlen_profile_read(int32_t idx, char* name, int32_t name_cap, int64_t* launches,
                        double* total_ms) {
  std::lock_guard<std::mutex> lock(vl::g_mu);
  // aggregate by name in first-seen order
  std::vector<std::string> order;
  std::map<std::string, std::pair<int64_t, double>> agg;
  for (auto& r : vl::g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return VL_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return VL_EHIP;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {1, double(ms)};
    } else {
      it->second.first += 1;
      it->second.second += double(ms);
    }
  }
  if (idx < 0 || size_t(idx) >= order.size()) return VL_EINVAL;
  const auto& nm = order[size_t(idx)];
  if (name && name_cap > 0) {
    std::strncpy(name, nm.c_str(), size_t(name_cap) - 1);
    name[name_cap - 1] = 0;
  }
  if (launches) *launches = agg[nm].first;
  if (total_ms) *total_ms = agg[nm].second;
  return VL_OK;
}

}  // extern "C"
