// Least-recently-used cache of the library's work lists (host side only: no
// HIP types, so the bookkeeping builds and is tested with a plain C++
// compiler).
//
// The window controller of "Asymmetric Attention Heads" (sections 5.3 and 5.8)
// picks new per-head windows at every control update (every fifth step in the
// pages' protocol), so a long run meets an open-ended sequence of window
// vectors.  The cache keeps at most `capacity` of them: looking an entry up
// makes it the most recently used, and inserting into a full cache hands the
// least recently used unpinned entry back to the caller, who releases its
// device memory.  Pinned entries (work lists that a captured HIP graph refers
// to) are never handed back; they stay until clear() and may push the cache
// past its capacity.
#pragma once

#include <cstddef>
#include <cstdint>
#include <list>
#include <map>
#include <utility>
#include <vector>

namespace aah {

template <class V>
class PlanLru {
 public:
  using Key = std::vector<int64_t>;

  explicit PlanLru(size_t capacity) : capacity_(capacity == 0 ? 1 : capacity) {}

  // The entry under key (now the most recently used), or nullptr.
  V* find(const Key& key) {
    auto it = index_.find(key);
    if (it == index_.end()) return nullptr;
    order_.splice(order_.begin(), order_, it->second);
    return &it->second->value;
  }

  // Marks the entry under key as pinned (never evicted).  Returns false if absent.
  bool pin(const Key& key) {
    auto it = index_.find(key);
    if (it == index_.end()) return false;
    it->second->pinned = true;
    return true;
  }

  // Inserts value under key (which must be absent) as the most recently used
  // entry and returns the entries evicted to make room: the least recently
  // used unpinned ones, as many as needed to keep size() <= capacity (fewer if
  // the rest are pinned).
  std::vector<V> insert(Key key, V value) {
    std::vector<V> evicted;
    while (index_.size() >= capacity_) {
      auto victim = order_.end();
      for (auto it = order_.end(); it != order_.begin();) {
        --it;
        if (!it->pinned) {
          victim = it;
          break;
        }
      }
      if (victim == order_.end()) break;  // everything left is pinned
      evicted.push_back(std::move(victim->value));
      index_.erase(victim->key);
      order_.erase(victim);
    }
    order_.push_front(Node{key, std::move(value), false});
    index_.emplace(std::move(key), order_.begin());
    return evicted;
  }

  // Removes every entry and returns them (pinned ones included), most recently used first.
  std::vector<V> clear() {
    std::vector<V> all;
    for (auto& n : order_) all.push_back(std::move(n.value));
    order_.clear();
    index_.clear();
    return all;
  }

  size_t size() const { return index_.size(); }
  size_t capacity() const { return capacity_; }

  // Keys from most to least recently used (for tests).
  std::vector<Key> keys() const {
    std::vector<Key> k;
    for (const auto& n : order_) k.push_back(n.key);
    return k;
  }

 private:
  struct Node {
    Key key;
    V value;
    bool pinned;
  };
  size_t capacity_;
  std::list<Node> order_;  // most recently used first
  std::map<Key, typename std::list<Node>::iterator> index_;
};

}  // namespace aah
