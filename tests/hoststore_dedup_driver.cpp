// Host-side driver of the page store's dedup resolution (paged_kv_cache_kvpool_amd/csrc/
// host_dedup.h) for tests/test_hoststore_dedup.py: pages are stood for by content ids, the
// injected hashes may collide at will, and "bytes equal" means equal content ids.
//
// stdin:  S (stored pages), then S lines "slot hash_a hash_b content";
//         N (blocks of the park call), then N lines "hash_a hash_b content"
// stdout: "rounds R" then N lines "stored id" (DedupRef of each block)
#include <cstdio>
#include <vector>

#include "../paged_kv_cache_kvpool_amd/csrc/host_dedup.h"

int main() {
  int s = 0, n = 0;
  if (scanf("%d", &s) != 1) return 2;
  kvp::PageIndex index;
  std::vector<long long> slot_content;
  for (int i = 0; i < s; ++i) {
    long long slot, c;
    unsigned long long a, b;
    if (scanf("%lld %llu %llu %lld", &slot, &a, &b, &c) != 4) return 2;
    if ((long long)slot_content.size() <= slot) slot_content.resize(slot + 1, -1);
    slot_content[slot] = c;
    index[kvp::PageHash{a, b}].push_back((int32_t)slot);
  }
  if (scanf("%d", &n) != 1) return 2;
  std::vector<kvp::PageHash> hv(n);
  std::vector<long long> content(n);
  for (int j = 0; j < n; ++j) {
    unsigned long long a, b;
    if (scanf("%llu %llu %lld", &a, &b, &content[j]) != 3) return 2;
    hv[j] = kvp::PageHash{a, b};
  }
  int rounds = 0;
  std::vector<kvp::DedupRef> ref;
  const int rc = kvp::dedup_resolve(hv, index, [&](const std::vector<kvp::DedupPair>& pairs,
                                                   std::vector<char>& equal) {
    ++rounds;
    for (size_t k = 0; k < pairs.size(); ++k) {
      const long long other = pairs[k].stored ? slot_content[pairs[k].id] : content[pairs[k].id];
      equal[k] = content[pairs[k].block] == other;
    }
    return 0;
  }, ref);
  if (rc) return 3;
  printf("rounds %d\n", rounds);
  for (int j = 0; j < n; ++j) printf("%d %d\n", ref[j].stored ? 1 : 0, ref[j].id);
  return 0;
}
