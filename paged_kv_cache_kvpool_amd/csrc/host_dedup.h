// Content deduplication of the pages parked in the host page store (NInfer serving doc,
// "Server options", --kv-host-cache-mib: pages shared by several sequences are stored once).
//
// A 128-bit content hash only nominates candidates: two pages are merged only after their bytes
// compare equal, so a hash collision (accidental or crafted) costs a comparison, never a wrong
// page.  Host logic only (no HIP): the library compares on the GPU, the CPU test of this file
// compares bytes on the host.
#pragma once

#include <stdint.h>

#include <unordered_map>
#include <vector>

namespace kvp {

struct PageHash {
  uint64_t a, b;
  bool operator==(const PageHash& o) const { return a == o.a && b == o.b; }
};
struct PageHashHasher {
  size_t operator()(const PageHash& h) const { return (size_t)(h.a ^ (h.b * 0x9E3779B97F4A7C15ull)); }
};
// Stored pages by hash: the slots of every stored page with that hash (more than one only after
// a collision).
using PageIndex = std::unordered_map<PageHash, std::vector<int32_t>, PageHashHasher>;

// What block j of a park call is: a page already in the store (stored, id = its slot) or a page
// new to the store whose content first appears at block id of the call (stored = false; the
// block with id == j is the one copied to the store).
struct DedupRef {
  bool stored;
  int32_t id;
};
// One comparison: block `block` of the call against a stored page (stored, id = slot) or against
// another block of the call (id = its index).
struct DedupPair {
  int32_t block;
  bool stored;
  int32_t id;
};

// Resolves the blocks of one park call, with hashes hv[0..n), against the store's pages and
// against each other.  compare(pairs, equal) fills equal[k] (1: the two contents are byte for
// byte the same) for every pair of the batch and returns 0, or an error code that is returned
// as is.  Each round, every unresolved block is compared with its next candidate (stored pages
// with its hash first, then the call's new pages with its hash, in block order); a block with no
// candidate left becomes a new page, and the blocks after it with the same hash take it as a
// candidate.  Without collisions a single round (one compare batch) settles every block, and
// blocks whose hash nothing else has need no comparison at all.
template <class Compare>
int dedup_resolve(const std::vector<PageHash>& hv, const PageIndex& index, Compare&& compare,
                  std::vector<DedupRef>& ref) {
  const int32_t n = (int32_t)hv.size();
  ref.assign(n, DedupRef{false, -1});
  // candidates per hash: stored slots, then new pages of this call as they appear
  std::unordered_map<PageHash, std::vector<DedupRef>, PageHashHasher> cands;
  for (int32_t j = 0; j < n; ++j) {
    auto it = cands.find(hv[j]);
    if (it != cands.end()) continue;
    std::vector<DedupRef>& c = cands[hv[j]];
    auto s = index.find(hv[j]);
    if (s != index.end())
      for (int32_t slot : s->second) c.push_back(DedupRef{true, slot});
  }
  std::vector<int32_t> next(n, 0);  // next candidate to try, per block
  std::vector<char> done(n, 0);
  std::vector<DedupPair> pairs;
  std::vector<char> equal;
  for (;;) {
    pairs.clear();
    for (int32_t j = 0; j < n; ++j) {
      if (done[j]) continue;
      std::vector<DedupRef>& c = cands[hv[j]];
      if (next[j] < (int32_t)c.size()) {
        const DedupRef& r = c[next[j]];
        pairs.push_back(DedupPair{j, r.stored, r.id});
      } else {
        // nothing left to compare with: block j holds a new page
        ref[j] = DedupRef{false, j};
        done[j] = 1;
        c.push_back(DedupRef{false, j});
      }
    }
    if (pairs.empty()) return 0;
    equal.assign(pairs.size(), 0);
    if (int rc = compare(pairs, equal)) return rc;
    for (size_t k = 0; k < pairs.size(); ++k) {
      const int32_t j = pairs[k].block;
      if (equal[k]) {
        ref[j] = DedupRef{pairs[k].stored, pairs[k].id};
        done[j] = 1;
      } else {
        ++next[j];
      }
    }
  }
}

}  // namespace kvp
