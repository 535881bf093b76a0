// Host check of the graph-cache bookkeeping (ae_graph_cache.h), following the
// behaviour the sglang PR 34599 summary lists for its bounded capture cache
// and prompt buckets (implementation items 3-5):
//  * a cache of capacity C holds at most C entries; a lookup refreshes an
//    entry, and a full cache hands back its least recently used entry;
//  * capacity 0 caches nothing;
//  * the bucket of a prompt length is the smallest configured length that
//    holds it, else the maximum length;
//  * bucket lists must be strictly increasing, within [1, max], and short.
// Prints the number of failed checks; exit status 0 when there are none.
#include "ae_graph_cache.h"

#include <cstdio>
#include <string>
#include <vector>

using namespace ae;

static int fails = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      ++fails;                                                \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);        \
    }                                                         \
  } while (0)

int main() {
  // LRU order and eviction
  {
    LruCache<CallKey, int> c(2);
    int ev = -1;
    CHECK(c.capacity() == 2 && c.size() == 0);
    CHECK(c.find({1, 10, 712}) == nullptr);
    CHECK(!c.insert({1, 10, 712}, 100, &ev));
    CHECK(!c.insert({1, 5, 712}, 200, &ev));
    CHECK(c.size() == 2);
    // touch the first: the second becomes least recently used
    CHECK(c.find({1, 10, 712}) && *c.find({1, 10, 712}) == 100);
    CHECK(c.insert({2, 10, 712}, 300, &ev));
    CHECK(ev == 200);
    CHECK(c.size() == 2);
    CHECK(c.find({1, 5, 712}) == nullptr);
    CHECK(c.find({2, 10, 712}) && *c.find({2, 10, 712}) == 300);
    // the key distinguishes the bucket
    CHECK(c.find({2, 10, 576}) == nullptr);
    // order: most recently used first
    const auto k = c.keys();
    CHECK(k.size() == 2 && k[0] == (CallKey{2, 10, 712}) && k[1] == (CallKey{1, 10, 712}));
    CHECK(c.insert({3, 3, 64}, 400, &ev) && ev == 100);
    const auto all = c.drain();
    CHECK(all.size() == 2 && all[0] == 400 && all[1] == 300);
    CHECK(c.size() == 0 && c.find({3, 3, 64}) == nullptr);
  }
  // a long random sequence against a plain reference list
  {
    const int cap = 5;
    LruCache<CallKey, int> c(cap);
    std::vector<std::pair<CallKey, int>> ref;  // most recent first
    unsigned x = 12345u;
    int evictions = 0, ref_evictions = 0;
    for (int i = 0; i < 20000; ++i) {
      x = x * 1664525u + 1013904223u;
      const CallKey k{static_cast<int>((x >> 8) % 4), static_cast<int>((x >> 16) % 3), 64};
      int* v = c.find(k);
      int ri = -1;
      for (size_t j = 0; j < ref.size(); ++j)
        if (ref[j].first == k) ri = static_cast<int>(j);
      CHECK((v != nullptr) == (ri >= 0));
      if (ri >= 0) {
        CHECK(*v == ref[ri].second);
        auto e = ref[ri];
        ref.erase(ref.begin() + ri);
        ref.insert(ref.begin(), e);
      } else {
        int ev = -1;
        if (c.insert(k, i, &ev)) {
          ++evictions;
          CHECK(ev == ref.back().second);
        }
        if (static_cast<int>(ref.size()) == cap) {
          ref.pop_back();
          ++ref_evictions;
        }
        ref.insert(ref.begin(), {k, i});
      }
      CHECK(c.size() == static_cast<int>(ref.size()) && c.size() <= cap);
    }
    CHECK(evictions == ref_evictions && evictions > 0);
  }
  // capacity 0 disables caching
  {
    LruCache<CallKey, int> c(0);
    int ev = -1;
    CHECK(c.insert({1, 1, 1}, 7, &ev) && ev == 7);
    CHECK(c.size() == 0 && c.find({1, 1, 1}) == nullptr);
  }
  // bucket choice
  {
    const std::vector<int> b = {256, 512, 768};
    CHECK(pick_bucket(b, 0, 1024) == 256);
    CHECK(pick_bucket(b, 1, 1024) == 256);
    CHECK(pick_bucket(b, 256, 1024) == 256);
    CHECK(pick_bucket(b, 257, 1024) == 512);
    CHECK(pick_bucket(b, 768, 1024) == 768);
    CHECK(pick_bucket(b, 769, 1024) == 1024);
    CHECK(pick_bucket({}, 5, 1024) == 1024);
  }
  // bucket validation
  {
    const int ok[3] = {64, 128, 712};
    const int dup[3] = {64, 64, 128};
    const int desc[2] = {128, 64};
    const int zero[2] = {0, 64};
    const int big[2] = {64, 713};
    CHECK(valid_buckets(ok, 3, 712, 32));
    CHECK(valid_buckets(nullptr, 0, 712, 32));
    CHECK(!valid_buckets(nullptr, 2, 712, 32));
    CHECK(!valid_buckets(dup, 3, 712, 32));
    CHECK(!valid_buckets(desc, 2, 712, 32));
    CHECK(!valid_buckets(zero, 2, 712, 32));
    CHECK(!valid_buckets(big, 2, 712, 32));
    CHECK(!valid_buckets(ok, 3, 712, 2));
    CHECK(!valid_buckets(ok, -1, 712, 32));
  }
  std::printf("failed checks: %d\n", fails);
  return fails == 0 ? 0 : 1;
}
