// Capacity-bounded cache of device work lists keyed by the cu_seqlens pattern
// (with the plan cache on, a call with a known pattern launches at once and
// can be captured in a HIP graph).  A plan fetched while the caller's stream
// is being captured is pinned: the graph keeps its device address, so the
// capacity eviction never frees it (only varlen_cache_clear does, on the
// caller's word that no graph still uses it).  When the cache is full, every
// unpinned plan is released; a cache full of pinned plans takes no new one.
//
// Pure C++ (no HIP): the values' device memory is released through a callback.
#pragma once
#include <stddef.h>

#include <map>
#include <string>

namespace vl {

template <class V>
class PlanCache {
 public:
  explicit PlanCache(size_t capacity) : cap_(capacity) {}

  // The cached value of `key`, or null; `pin` marks it as held by a graph.
  V* find(const std::string& key, bool pin) {
    auto it = map_.find(key);
    if (it == map_.end()) return nullptr;
    it->second.pinned = it->second.pinned || pin;
    return &it->second.value;
  }

  // Makes room for one more entry: when full, every unpinned entry is passed
  // to release(value) and dropped.  Returns false (and drops nothing) when the
  // cache is full of pinned entries.
  template <class F>
  bool make_room(F release) {
    if (map_.size() < cap_) return true;
    size_t pinned = 0;
    for (const auto& kv : map_) pinned += kv.second.pinned ? 1 : 0;
    if (pinned >= cap_) return false;
    for (auto it = map_.begin(); it != map_.end();) {
      if (it->second.pinned) {
        ++it;
      } else {
        release(it->second.value);
        it = map_.erase(it);
      }
    }
    return true;
  }

  void insert(const std::string& key, const V& value, bool pin) {
    map_[key] = Entry{value, pin};
  }

  // Drops everything, pinned entries included.
  template <class F>
  void clear(F release) {
    for (auto& kv : map_) release(kv.second.value);
    map_.clear();
  }

  size_t size() const { return map_.size(); }
  bool pinned(const std::string& key) const {
    auto it = map_.find(key);
    return it != map_.end() && it->second.pinned;
  }

 private:
  struct Entry {
    V value;
    bool pinned = false;
  };
  size_t cap_;
  std::map<std::string, Entry> map_;
};

}  // namespace vl
