// Host block manager under AddressSanitizer and UndefinedBehaviorSanitizer:
// a seeded churn of add / fork / append (copy-on-write) / free / swap-out /
// swap-in with the invariant check after every operation, plus the error
// paths (bad ids, OOM, short output buffers).  Exit status 0 = clean.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

namespace pkv {
// the library's error reporter lives in its HIP layer; a plain one here
pkv_status fail(pkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return s;
}
}  // namespace pkv

#define CHECK(x)                                                  \
  do {                                                            \
    if (!(x)) {                                                   \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #x); \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main() {
  for (int B : {1, 4, 16}) {
    const int NB = 96, NC = 64;
    std::mt19937 rng(1234 + B);
    std::vector<int32_t> order(NB);
    for (int i = 0; i < NB; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pkv_block_manager* bm = nullptr;
    CHECK(pkv_bm_create(NB, B, order.data(), &bm) == PKV_OK);
    CHECK(pkv_bm_set_cpu_blocks(bm, NC) == PKV_OK);
    std::vector<int32_t> live, swapped;
    std::vector<int64_t> pairs(2 * (NB + NC));
    std::vector<int32_t> table(NB + 1);
    std::vector<int64_t> slots(4 * NB);
    for (int step = 0; step < 4000; ++step) {
      const int op = (int)(rng() % 7);
      pkv_status st = PKV_OK;
      int32_t id = -1, n = 0;
      if (op == 0 || live.empty()) {
        st = pkv_bm_add_seq(bm, (int32_t)(rng() % (3 * B + 5)), &id);
        if (st == PKV_OK) live.push_back(id);
      } else {
        const size_t k = rng() % live.size();
        const int32_t s = live[k];
        bool is_swapped = false;
        for (int32_t x : swapped) is_swapped |= (x == s);
        if (op == 1) {
          st = pkv_bm_fork(bm, s, &id);
          if (st == PKV_OK) live.push_back(id);
          else CHECK(is_swapped || st == PKV_ERR_OOM);
        } else if (op == 2) {
          CHECK(pkv_bm_free_seq(bm, s) == PKV_OK);
          live.erase(live.begin() + (long)k);
          for (size_t j = 0; j < swapped.size(); ++j)
            if (swapped[j] == s) swapped.erase(swapped.begin() + (long)j);
        } else if (op == 3) {
          int64_t slot;
          int32_t src, dst;
          st = pkv_bm_append_token(bm, s, &slot, &src, &dst);
          if (st == PKV_OK) CHECK(slot >= 0 && slot < (int64_t)NB * B && (src < 0) == (dst < 0));
        } else if (op == 4) {
          st = pkv_bm_swap_out(bm, s, pairs.data(), (int32_t)pairs.size() / 2, &n);
          if (st == PKV_OK) swapped.push_back(s);
        } else if (op == 5) {
          if (!swapped.empty()) {
            const size_t j = rng() % swapped.size();
            st = pkv_bm_swap_in(bm, swapped[j], pairs.data(), (int32_t)pairs.size() / 2, &n);
            if (st == PKV_OK) swapped.erase(swapped.begin() + (long)j);
          }
        } else {
          int32_t len = 0;
          CHECK(pkv_bm_seq_len(bm, s, &len) == PKV_OK);
          if (!is_swapped) {
            CHECK(pkv_bm_table(bm, s, table.data(), (int32_t)table.size(), &n) == PKV_OK);
            CHECK(n == (len + B - 1) / B);
            if (len > 0) CHECK(pkv_bm_slots(bm, s, 0, len, slots.data()) == PKV_OK);
            for (int32_t i = 0; i < n; ++i) {
              int32_t rc = 0;
              CHECK(pkv_bm_refcount(bm, table[i], &rc) == PKV_OK && rc >= 1);
            }
            // a buffer one entry short is refused, an out-of-range slot query too
            if (n > 0) CHECK(pkv_bm_table(bm, s, table.data(), n - 1, &n) != PKV_OK);
            CHECK(pkv_bm_slots(bm, s, len, 1, slots.data()) != PKV_OK);
          }
        }
        CHECK(st == PKV_OK || st == PKV_ERR_OOM || st == PKV_ERR_INVALID_ARG);
      }
      CHECK(pkv_bm_check(bm) == PKV_OK);
    }
    int32_t tmp;
    CHECK(pkv_bm_fork(bm, 1 << 20, &tmp) != PKV_OK);   // unknown ids
    CHECK(pkv_bm_free_seq(bm, -1) != PKV_OK);
    CHECK(pkv_bm_refcount(bm, NB, &tmp) != PKV_OK);
    pkv_bm_destroy(bm);
  }
  pkv_block_manager* bm = nullptr;
  CHECK(pkv_bm_create(-1, 16, nullptr, &bm) != PKV_OK && bm == nullptr);
  const int32_t not_perm[3] = {0, 2, 2};
  CHECK(pkv_bm_create(3, 16, not_perm, &bm) != PKV_OK && bm == nullptr);
  CHECK(pkv_bm_create(0, 16, nullptr, &bm) == PKV_OK);   // an empty pool: every add is OOM
  int32_t id = 0;
  CHECK(pkv_bm_add_seq(bm, 1, &id) == PKV_ERR_OOM && pkv_bm_check(bm) == PKV_OK);
  pkv_bm_destroy(bm);
  std::puts("bm_churn clean");
  return 0;
}
