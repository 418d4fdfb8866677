// Randomised allocator session for the AddressSanitizer / UBSan build of the host
// allocator: alloc, alloc_batch, fork, free and queries in random order, checking the
// allocator's invariants after every step.  Exits non-zero on a broken invariant.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c); \
      std::exit(2);                                                   \
    }                                                                 \
  } while (0)

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 200;
  std::mt19937 rng(12345);
  for (int r = 0; r < rounds; ++r) {
    const int N = 1 + rng() % 40, B = 1 << (rng() % 5);
    std::vector<int32_t> order(N);
    for (int i = 0; i < N; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pkv_allocator* a = nullptr;
    CHECK(pkv_allocator_create(N, B, order.data(), &a) == PKV_OK);
    std::set<int64_t> live;
    for (int step = 0; step < 300; ++step) {
      const int op = rng() % 6;
      const int64_t s = rng() % 8, t = rng() % 8;
      const int n = rng() % 50;
      if (op <= 1) {
        std::vector<int64_t> slots(n + 1);
        int32_t pair[2], nc = 0;
        if (pkv_alloc(a, s, n, slots.data(), pair, &nc) == PKV_OK) live.insert(s);
      } else if (op == 2) {
        int64_t ids[3] = {s, (s + 1) % 8, (s + 3) % 8};
        std::vector<int64_t> slots(3 * 4);
        int32_t pairs[6], nc = 0;
        if (pkv_alloc_batch(a, ids, 3, 4, slots.data(), pairs, &nc) == PKV_OK)
          for (auto id : ids) live.insert(id);
      } else if (op == 3) {
        if (pkv_fork(a, s, t, static_cast<int32_t>(rng() % 60) - 1) == PKV_OK) live.insert(t);
      } else if (op == 4) {
        if (pkv_free(a, s) == PKV_OK) live.erase(s);
      } else {
        pkv_stats st;
        CHECK(pkv_allocator_stats(a, &st) == PKV_OK);
        CHECK(st.free_blocks + st.allocated_blocks == N);
      }
      // references = occurrences in tables; free list + referenced = pool
      std::vector<int> count(N, 0);
      for (int64_t id : live) {
        int32_t nb = 0, len = 0;
        CHECK(pkv_get_block_table(a, id, nullptr, 0, &nb, &len) == PKV_OK);
        CHECK(nb == (len + B - 1) / B);
        std::vector<int32_t> tab(nb + 1);
        CHECK(pkv_get_block_table(a, id, tab.data(), nb, nullptr, nullptr) == PKV_OK);
        for (int i = 0; i < nb; ++i) {
          CHECK(tab[i] >= 0 && tab[i] < N);
          ++count[tab[i]];
        }
      }
      int32_t nf = 0;
      CHECK(pkv_free_list(a, nullptr, 0, &nf) == PKV_OK);
      std::vector<int32_t> fl(nf + 1);
      CHECK(pkv_free_list(a, fl.data(), nf, nullptr) == PKV_OK);
      std::vector<int> onfree(N, 0);
      for (int i = 0; i < nf; ++i) {
        CHECK(onfree[fl[i]] == 0);
        onfree[fl[i]] = 1;
      }
      for (int b = 0; b < N; ++b) {
        CHECK(pkv_block_ref_count(a, b) == count[b]);
        CHECK((count[b] == 0) == (onfree[b] == 1));
      }
    }
    for (int64_t id : live) CHECK(pkv_free(a, id) == PKV_OK);
    int32_t nf = 0;
    CHECK(pkv_free_list(a, nullptr, 0, &nf) == PKV_OK && nf == N);
    pkv_allocator_destroy(a);
  }
  std::puts("ok");
  return 0;
}
