// Randomized stress of the host block allocator, built with sanitizers by
// tests/test_allocator.py.  After every operation the allocator's view (tables,
// lengths, reference counts, free count) is checked against a shadow model.
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
  for (int step = 0; step < 20000; ++step) {
    const int op = static_cast<int>(rng() % 11);
    if (op < 3) {
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
    }
    CHECK(pkv_alloc_num_free(a) == N - used);
    CHECK(pkv_alloc_num_seqs(a) == static_cast<int32_t>(lens.size()));
  }
  pkv_alloc_destroy(a);
  std::printf("ok\n");
  return 0;
}
