// Unit test of the work-list cache's bookkeeping (head_causal_local_amd/csrc/plan_cache.hpp), built with a
// plain C++ compiler (under AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_build.py).
// Prints "ok" and exits 0 when every check passes.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "plan_cache.hpp"

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

using Key = std::vector<int64_t>;

int main() {
  // Least recently used goes first; a lookup refreshes an entry.
  {
    aah::PlanLru<std::string> c(3);
    CHECK(c.insert({1}, "a").empty());
    CHECK(c.insert({2}, "b").empty());
    CHECK(c.insert({3}, "c").empty());
    CHECK(c.find({1}) != nullptr && *c.find({1}) == "a");  // 1 is now the most recent
    auto ev = c.insert({4}, "d");
    CHECK(ev.size() == 1 && ev[0] == "b");
    CHECK(c.size() == 3 && c.find({2}) == nullptr);
    CHECK((c.keys() == std::vector<Key>{{4}, {1}, {3}}));
    ev = c.insert({5}, "e");
    CHECK(ev.size() == 1 && ev[0] == "c");
  }
  // Pinned entries are never evicted, even when that leaves the cache over capacity.
  {
    aah::PlanLru<int> c(2);
    c.insert({10}, 10);
    CHECK(c.pin({10}) && !c.pin({99}));
    c.insert({11}, 11);
    auto ev = c.insert({12}, 12);
    CHECK(ev.size() == 1 && ev[0] == 11);
    CHECK(c.find({10}) != nullptr);
    c.pin({12});
    ev = c.insert({13}, 13);  // both older entries pinned: nothing to evict
    CHECK(ev.empty() && c.size() == 3);
    ev = c.insert({14}, 14);  // 13 is the only unpinned one
    CHECK(ev.size() == 1 && ev[0] == 13 && c.size() == 3);
    auto all = c.clear();
    CHECK(all.size() == 3 && c.size() == 0);
  }
  // A long run of distinct window vectors (a controller choosing new windows at every update): the cache
  // never holds more than its capacity, every entry it evicts was inserted once and is released once, and
  // the most recent `capacity` vectors are all still found.
  {
    const size_t cap = 64;
    aah::PlanLru<int> c(cap);
    std::mt19937 rng(7);
    std::uniform_int_distribution<int> pick(0, 3);
    const int cand[4] = {512, 1024, 2048, 4096};
    std::vector<Key> inserted;
    std::set<Key> seen;
    std::multiset<int> released;
    for (int i = 0; i < 2000; ++i) {
      Key k = {0, 0, 4, 32, 32, 4096};
      for (int h = 0; h < 32; ++h) k.push_back(cand[pick(rng)]);
      if (!seen.insert(k).second) continue;
      CHECK(c.find(k) == nullptr);
      for (int v : c.insert(k, static_cast<int>(inserted.size()))) released.insert(v);
      inserted.push_back(k);
      CHECK(c.size() <= cap);
    }
    CHECK(inserted.size() > 1000);
    CHECK(released.size() == inserted.size() - cap);
    for (size_t j = 0; j < released.size(); ++j) CHECK(released.count(static_cast<int>(j)) == 1);
    for (size_t j = inserted.size() - cap; j < inserted.size(); ++j) CHECK(c.find(inserted[j]) != nullptr);
  }
  std::printf("ok\n");
  return 0;
}
