// Host-side bookkeeping of captured denoise-call graphs: a bounded cache
// keyed by the call's signature with least-recently-used eviction, and the
// choice of a prefix-length bucket.
//
// Follows the sglang PR 34599 summary, implementation items 3-5: captured
// action graphs live in a bounded cache ordered by last use; an entry's graph
// is released before the entry is replaced or evicted; when the cache is full
// the exact mode runs a signature it has not seen without capturing it (the
// other mode evicts the least recently used entry); a capacity of zero turns
// capture off; hits, misses and evictions are counted.  Opt-in prompt
// bucketing pads a prompt on the right, masked, to the smallest configured
// length that holds it, so one graph serves every prompt of a bucket; the
// bucket lengths must be positive, strictly increasing and no longer than the
// maximum length.
//
// Plain C++ (no HIP types), so the logic is checked on the host.
#pragma once

#include <algorithm>
#include <list>
#include <map>
#include <utility>
#include <vector>

namespace ae {

// What a captured denoise call depends on besides device data: the batch,
// the Euler step count and the prefix bucket (which sizes the attention's
// key splits).
struct CallKey {
  int batch, steps, bucket;
  bool operator<(const CallKey& o) const {
    if (batch != o.batch) return batch < o.batch;
    if (steps != o.steps) return steps < o.steps;
    return bucket < o.bucket;
  }
  bool operator==(const CallKey& o) const {
    return batch == o.batch && steps == o.steps && bucket == o.bucket;
  }
};

template <typename K, typename V>
class LruCache {
 public:
  explicit LruCache(int capacity = 0) : cap_(std::max(0, capacity)) {}

  int capacity() const { return cap_; }
  int size() const { return static_cast<int>(order_.size()); }

  // The value cached under k (and k becomes the most recently used), or
  // nullptr.
  V* find(const K& k) {
    auto it = index_.find(k);
    if (it == index_.end()) return nullptr;
    order_.splice(order_.begin(), order_, it->second);
    return &it->second->second;
  }

  // Cache v under k (k must not be cached).  When the cache is full the
  // least recently used entry is removed and handed back through *evicted
  // (the caller releases it); returns whether that happened.  With capacity
  // 0 nothing is cached: v itself comes back as evicted.
  bool insert(const K& k, V v, V* evicted) {
    if (cap_ == 0) {
      *evicted = v;
      return true;
    }
    bool ev = false;
    if (size() >= cap_) {
      auto last = std::prev(order_.end());
      *evicted = last->second;
      index_.erase(last->first);
      order_.erase(last);
      ev = true;
    }
    order_.emplace_front(k, v);
    index_[k] = order_.begin();
    return ev;
  }

  // Every cached value, most recently used first; the cache is emptied.
  std::vector<V> drain() {
    std::vector<V> out;
    for (auto& kv : order_) out.push_back(kv.second);
    order_.clear();
    index_.clear();
    return out;
  }

  // Keys from most to least recently used.
  std::vector<K> keys() const {
    std::vector<K> out;
    for (const auto& kv : order_) out.push_back(kv.first);
    return out;
  }

 private:
  using Entry = std::pair<K, V>;
  int cap_;
  std::list<Entry> order_;
  std::map<K, typename std::list<Entry>::iterator> index_;
};

// The smallest bucket length >= prefix_len among `buckets` (ascending), or
// max_len when none holds it (the capacity is the implicit last bucket).
inline int pick_bucket(const std::vector<int>& buckets, int prefix_len, int max_len) {
  for (int b : buckets)
    if (b >= prefix_len) return b;
  return max_len;
}

// A bucket list is valid when it is strictly ascending, every length is in
// [1, max_len] and there are at most max_n of them.
inline bool valid_buckets(const int* lens, int n, int max_len, int max_n) {
  if (n < 0 || n > max_n || (n > 0 && !lens)) return false;
  for (int i = 0; i < n; ++i) {
    if (lens[i] < 1 || lens[i] > max_len) return false;
    if (i > 0 && lens[i] <= lens[i - 1]) return false;
  }
  return true;
}

}  // namespace ae
