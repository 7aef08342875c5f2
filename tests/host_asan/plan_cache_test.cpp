// Unit test of the plan cache's eviction rule (plan_cache.h), built and run on
// the host with the sanitizers by tests/test_host_sanitizers.py.  Exits 0 when
// every check holds; prints the failed check and exits 1 otherwise.
#include <cstdio>
#include <set>
#include <string>

#include "plan_cache.h"

namespace {
int failures = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s\n", what);
    ++failures;
  }
}
}  // namespace

int main() {
  std::multiset<int> released;
  auto release = [&](int& v) { released.insert(v); };
  vl::PlanCache<int> c(4);
  c.insert("a", 1, false);
  c.insert("b", 2, false);
  c.insert("c", 3, false);
  check(c.make_room(release) && released.empty(), "room below capacity frees nothing");
  c.insert("d", 4, false);
  // a captured graph uses b and d: pinned on the hit
  check(c.find("b", true) && *c.find("b", false) == 2, "hit returns the value");
  check(c.find("d", true) != nullptr, "hit on d");
  check(c.pinned("b") && c.pinned("d") && !c.pinned("a"), "pins set by hits under capture");
  check(c.find("zz", true) == nullptr, "miss returns null");
  // full: the unpinned a and c go, the pinned b and d stay
  check(c.make_room(release), "full cache with unpinned plans makes room");
  check(c.size() == 2 && released == std::multiset<int>{1, 3}, "only unpinned plans released");
  check(c.find("b", false) && c.find("d", false), "pinned plans survive eviction");
  check(!c.find("a", false) && !c.find("c", false), "evicted plans are gone");
  // a pin is never dropped by a later hit outside capture
  c.find("b", false);
  check(c.pinned("b"), "pin persists");
  // fill with pinned plans: no room, nothing released
  c.insert("e", 5, true);
  c.insert("f", 6, true);
  released.clear();
  check(!c.make_room(release) && released.empty() && c.size() == 4,
        "a cache full of pinned plans refuses and frees nothing");
  // clear drops everything
  c.clear(release);
  check(c.size() == 0 && released.size() == 4, "clear releases pinned plans too");
  check(c.make_room(release), "room after clear");
  if (failures == 0) std::printf("plan cache: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
