// Randomized stress of the host block allocator, built with sanitizers by
// tests/test_allocator.py.  After every operation the allocator's view (tables,
// lengths, reference counts, free count) is checked against a shadow model.
// Prompts admitted by token ids (prefix caching) are checked against the
// shadow's record of what each block holds: a block shared by a match must
// hold exactly the new prompt's tokens up to its end, whether it was live or
// a freed block not yet reused, under eviction pressure from the other
// operations.
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv_alloc.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::printf("check failed line %d: %s\n", __LINE__, #c);          \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

int main() {
  const int N = 400, BS = 16, MAXB = N;
  pkv_alloc* a = pkv_alloc_create(N, BS, 77);
  CHECK(a != nullptr);
  std::mt19937_64 rng(1);
  std::map<int64_t, int> lens;  // shadow: seq -> tokens
  int64_t next_id = 0;
  std::vector<int32_t> table(MAXB);
  // shadow of block contents: the token prefix a block's K/V stands for (the
  // prompt's tokens up to the block's end), empty when unknown
  std::vector<std::vector<int32_t>> content(N);
  std::vector<int32_t> before(N);
  int revived = 0, evicted = 0;  // matches of freed blocks; cache entries reused for other contents
  for (int step = 0; step < 20000; ++step) {
    for (int b = 0; b < N; ++b) before[b] = pkv_alloc_refcount(a, b);
    const int cached_before = pkv_alloc_num_cached(a);
    bool prefix_op = false;
    const int op = static_cast<int>(rng() % 14);
    if (op >= 12) {
      // a prompt of 0-5 full blocks named from a 3-letter alphabet, and a tail
      prefix_op = true;
      std::vector<int32_t> toks;
      const int nb = static_cast<int>(rng() % 6);
      for (int j = 0; j < nb; ++j) {
        const int name = static_cast<int>(rng() % 3);
        for (int i = 0; i < BS; ++i) toks.push_back(1000 * name + i);
      }
      const int tail = static_cast<int>(rng() % BS);
      for (int i = 0; i < tail; ++i) toks.push_back(7 + i);
      int32_t cached = -1;
      const int rc = pkv_alloc_add_seq_prefix(a, next_id, toks.empty() ? nullptr : toks.data(),
                                              static_cast<int32_t>(toks.size()), &cached);
      if (rc == PKV_OK) {
        const int n = static_cast<int>(toks.size());
        lens[next_id] = n;
        CHECK(cached >= 0 && cached % BS == 0 && cached <= nb * BS);
        int32_t L;
        CHECK(pkv_alloc_block_tables(a, &next_id, 1, MAXB, -1, table.data(), &L) == PKV_OK && L == n);
        for (int j = 0; j < (n + BS - 1) / BS; ++j) {
          std::vector<int32_t> chain(toks.begin(), toks.begin() + std::min(n, (j + 1) * BS));
          if (j < cached / BS) {
            CHECK(content[table[j]] == chain);  // exact: the block holds these tokens' K/V
            revived += before[table[j]] == 0;
          } else {
            CHECK(before[table[j]] == 0);  // a fresh block
            content[table[j]] = j < nb ? chain : std::vector<int32_t>();
          }
        }
      } else {
        CHECK(rc == PKV_E_NOMEM);
      }
      ++next_id;
    } else if (op < 3) {
      const int n = static_cast<int>(rng() % 300);
      const int rc = pkv_alloc_add_seq(a, next_id, n);
      if (rc == PKV_OK) lens[next_id] = n;
      else CHECK(rc == PKV_E_NOMEM);
      ++next_id;
    } else if (op < 4 && !lens.empty()) {
      auto it = lens.begin();
      std::advance(it, rng() % lens.size());
      const int share = static_cast<int>(it->second / BS);
      const int n = share * BS + static_cast<int>(rng() % 40);
      const int rc = pkv_alloc_add_seq_shared(a, next_id, n, it->first, share);
      if (rc == PKV_OK) lens[next_id] = n;
      else CHECK(rc == PKV_E_NOMEM);
      ++next_id;
    } else if (op < 5 && lens.size() >= 2) {
      // share a prefix between two live sequences
      auto d = lens.begin(), sr = lens.begin();
      std::advance(d, rng() % lens.size());
      std::advance(sr, rng() % lens.size());
      const int most = std::min(d->second, sr->second) / BS;
      const int n = static_cast<int>(rng() % (most + 2));  // sometimes one too many
      const int rc = pkv_alloc_share_prefix(a, d->first, sr->first, n);
      if (d->first == sr->first || n > most) CHECK(rc == PKV_E_SHAPE);
      else CHECK(rc == PKV_OK);
    } else if (op < 8 && !lens.empty()) {
      std::vector<int64_t> ids;
      for (auto& kv : lens)
        if (rng() % 2) ids.push_back(kv.first);
      std::vector<int64_t> slots(ids.size());
      const int rc = pkv_alloc_append_slots(a, ids.data(), static_cast<int32_t>(ids.size()), slots.data());
      if (rc == PKV_OK) {
        std::set<int64_t> uniq(slots.begin(), slots.end());
        CHECK(uniq.size() == slots.size());
        for (size_t i = 0; i < ids.size(); ++i) {
          const int pos = lens[ids[i]]++;
          CHECK(pkv_alloc_block_tables(a, &ids[i], 1, MAXB, -1, table.data(), nullptr) == PKV_E_NULL);
          int32_t L;
          CHECK(pkv_alloc_block_tables(a, &ids[i], 1, MAXB, -1, table.data(), &L) == PKV_OK);
          CHECK(L == pos + 1);
          CHECK(slots[i] == static_cast<int64_t>(table[pos / BS]) * BS + pos % BS);
          CHECK(pkv_alloc_refcount(a, table[pos / BS]) == 1);  // never a shared block
        }
      } else {
        CHECK(rc == PKV_E_NOMEM);
      }
    } else if (!lens.empty()) {
      auto it = lens.begin();
      std::advance(it, rng() % lens.size());
      CHECK(pkv_alloc_free_seq(a, it->first) == PKV_OK);
      lens.erase(it);
    }
    // invariants: refcount of every block == number of holders; free count
    std::vector<int> holders(N, 0);
    for (auto& kv : lens) {
      int32_t L;
      const int64_t id = kv.first;
      if ((kv.second + BS - 1) / BS > MAXB) continue;
      CHECK(pkv_alloc_block_tables(a, &id, 1, MAXB, -1, table.data(), &L) == PKV_OK);
      CHECK(L == kv.second);
      const int nb = (L + BS - 1) / BS;
      for (int j = 0; j < nb; ++j) {
        CHECK(table[j] >= 0 && table[j] < N);
        ++holders[table[j]];
      }
      for (int j = nb; j < MAXB; ++j) CHECK(table[j] == -1);
    }
    int used = 0;
    for (int b = 0; b < N; ++b) {
      CHECK(pkv_alloc_refcount(a, b) >= holders[b]);
      if (pkv_alloc_refcount(a, b) > 0) ++used;
      // a block handed out by any other operation holds new, unknown contents
      if (!prefix_op && before[b] == 0 && pkv_alloc_refcount(a, b) > 0) content[b].clear();
    }
    CHECK(pkv_alloc_num_free(a) == N - used);
    CHECK(pkv_alloc_num_cached(a) >= 0 && pkv_alloc_num_cached(a) <= pkv_alloc_num_free(a));
    if (op >= 3 && op < 8 && pkv_alloc_num_cached(a) < cached_before) ++evicted;
    CHECK(pkv_alloc_num_seqs(a) == static_cast<int32_t>(lens.size()));
  }
  pkv_alloc_destroy(a);
  // the run must have exercised both sides of the cache
  CHECK(revived > 20 && evicted > 50);
  std::printf("ok (%d freed blocks matched again, %d operations reused cached blocks)\n", revived, evicted);
  return 0;
}
