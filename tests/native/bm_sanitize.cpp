// Randomised driver of the host block manager (block_manager.cpp) for a
// sanitizer build: every entry point, its error paths, and after every step
// the invariants the manager promises (each block's count equals its
// occurrences in the tables of sequences on the device, free blocks are
// exactly those with count 0, a table holds ceil(L / B) blocks).  Exit code 0
// means every check held; the sanitizers abort on any memory or undefined-
// behaviour error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

static int fail(const char* what, int line) {
  fprintf(stderr, "check failed at line %d: %s\n", line, what);
  exit(1);
}
#define CHECK(c) ((c) ? (void)0 : (void)fail(#c, __LINE__))

int main(int argc, char** argv) {
  const int seeds = argc > 1 ? atoi(argv[1]) : 40;
  // bad sizes
  CHECK(pkv_bm_create(0, 16, 4) == nullptr);
  CHECK(pkv_bm_create(16, 0, 4) == nullptr);
  CHECK(pkv_bm_create(16, 16, 0) == nullptr);
  CHECK(pkv_bm_create(0x7fffffff, 16, 4) == nullptr);
  pkv_bm_destroy(nullptr);
  for (int seed = 0; seed < seeds; ++seed) {
    std::mt19937 rng(1000 + seed);
    const int NB = 8 + (int)(rng() % 120), B = (rng() % 2) ? 16 : 4, MB = 2 + (int)(rng() % 12);
    pkv_block_manager* m = pkv_bm_create(NB, B, MB);
    CHECK(m != nullptr);
    std::set<int32_t> live, swapped;
    std::map<int32_t, std::vector<int32_t>> saved;  // swapped sequence -> its blocks when it left
    int32_t next_id = 0;
    for (int step = 0; step < 400; ++step) {
      const int op = (int)(rng() % 10);
      std::vector<int32_t> ids(live.begin(), live.end());
      const int32_t pick = ids.empty() ? -1 : ids[rng() % ids.size()];
      if (op == 0 || ids.empty()) {
        int32_t s = -5;
        CHECK(pkv_bm_add_sequence(m, &s) == PKV_OK);
        CHECK(s == next_id++);
        live.insert(s);
      } else if (op == 1) {
        int32_t c = -5;
        CHECK(pkv_bm_fork(m, pick, &c) == PKV_OK);
        CHECK(c == next_id++);
        live.insert(c);
      } else if (op == 2 && ids.size() > 2) {
        CHECK(pkv_bm_free(m, pick) == PKV_OK);
        live.erase(pick);
      } else if (op <= 5) {
        const int n = (int)(rng() % (2 * B + 2));
        std::vector<int32_t> slots(n + 1, -7);
        int32_t src = -7, dst = -7, nc = -7;
        const int st = pkv_bm_append(m, pick, n, slots.data(), &src, &dst, &nc);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
        if (st == PKV_OK) {
          CHECK(nc == 0 || nc == 1);
          for (int i = 0; i < n; ++i) CHECK(slots[i] >= 0 && slots[i] < NB * B);
          if (nc == 1) CHECK(src >= 0 && src < NB && dst >= 0 && dst < NB && src != dst);
        }
      } else if (op == 6) {
        std::vector<int32_t> seqs(ids.begin(), ids.end());
        const int n = (int)seqs.size();
        std::vector<int32_t> slots(n + 1), src(n + 1), dst(n + 1);
        int32_t nc = -1, nd = -1;
        const int st = pkv_bm_append_batch(m, seqs.data(), n, slots.data(), src.data(), dst.data(), &nc, &nd);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
        CHECK(nd >= 0 && nd <= n && nc >= 0 && nc <= nd);
        if (st == PKV_OK) CHECK(nd == n);
      } else if (op == 7 && ids.size() > 1) {
        std::vector<int32_t> blk(MB + 1);
        int32_t nb = -1;
        CHECK(pkv_bm_swap_out(m, pick, blk.data(), MB, &nb) == PKV_OK);
        CHECK(nb >= 0 && nb <= MB);
        saved[pick] = std::vector<int32_t>(blk.begin(), blk.begin() + nb);
        live.erase(pick);
        swapped.insert(pick);
        // a swapped sequence cannot append, fork or swap out again
        int32_t s1[2], a = 0, b2 = 0, n2 = 0, c = 0;
        CHECK(pkv_bm_append(m, pick, 1, s1, &a, &b2, &n2) == PKV_ERR_BAD_SEQUENCE);
        CHECK(pkv_bm_fork(m, pick, &c) == PKV_ERR_BAD_SEQUENCE);
        CHECK(pkv_bm_swap_out(m, pick, blk.data(), MB, &nb) == PKV_ERR_BAD_SEQUENCE);
      } else if (op == 8 && !swapped.empty()) {
        const int32_t s = *swapped.begin();
        std::vector<int32_t> blk(MB + 1);
        int32_t nb = -1;
        const int st = pkv_bm_swap_in(m, s, blk.data(), MB, &nb);
        CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
        if (st == PKV_OK) {
          CHECK(nb == (int32_t)saved[s].size());
          swapped.erase(s);
          live.insert(s);
        } else if (rng() % 2) {
          CHECK(pkv_bm_free(m, s) == PKV_OK);
          swapped.erase(s);
        }
      } else {
        // error paths: unknown ids, negative counts, a table buffer too small
        int32_t x = 0, y = 0, z = 0, w = 0;
        CHECK(pkv_bm_fork(m, -1, &x) == PKV_ERR_BAD_SEQUENCE);
        CHECK(pkv_bm_fork(m, next_id + 3, &x) == PKV_ERR_BAD_SEQUENCE);
        CHECK(pkv_bm_free(m, next_id + 9) == PKV_ERR_BAD_SEQUENCE);
        CHECK(pkv_bm_append(m, pick, -2, &x, &y, &z, &w) != PKV_OK);
        CHECK(pkv_bm_ref_count(m, -1, &x) != PKV_OK);
        CHECK(pkv_bm_ref_count(m, NB, &x) != PKV_OK);
        int32_t one = 0, nb = 0;
        int64_t len = 0;
        const int st = pkv_bm_table(m, pick, &one, 0, &nb, &len);
        CHECK(st == PKV_OK || st == PKV_ERR_SHAPE);
        // missing out-parameters are reported, never dereferenced
        CHECK(pkv_bm_add_sequence(m, nullptr) == PKV_ERR_NULL);
        CHECK(pkv_bm_fork(m, pick, nullptr) == PKV_ERR_NULL);
        CHECK(pkv_bm_append(m, pick, 1, nullptr, &y, &z, &w) == PKV_ERR_NULL);
        CHECK(pkv_bm_append(m, pick, 1, &x, &y, &z, nullptr) == PKV_ERR_NULL);
        CHECK(pkv_bm_append_batch(m, nullptr, 1, &x, &y, &z, &w, &one) == PKV_ERR_NULL);
        CHECK(pkv_bm_table(m, pick, &one, 1, nullptr, &len) == PKV_ERR_NULL);
        CHECK(pkv_bm_ref_count(m, 0, nullptr) == PKV_ERR_NULL);
        CHECK(pkv_bm_usage(m, nullptr, nullptr, nullptr, nullptr) == PKV_ERR_NULL);
        CHECK(pkv_bm_free(nullptr, pick) == PKV_ERR_NULL);
      }
      // invariants
      std::vector<int> occ(NB, 0);
      for (int32_t s : live) {
        std::vector<int32_t> blk(MB);
        int32_t nb = -1;
        int64_t len = -1;
        CHECK(pkv_bm_table(m, s, blk.data(), MB, &nb, &len) == PKV_OK);
        CHECK(nb == (int32_t)((len + B - 1) / B));
        for (int i = 0; i < nb; ++i) {
          CHECK(blk[i] >= 0 && blk[i] < NB);
          occ[blk[i]]++;
        }
      }
      int zero = 0;
      for (int b = 0; b < NB; ++b) {
        int32_t r = -1;
        CHECK(pkv_bm_ref_count(m, b, &r) == PKV_OK);
        CHECK(r == occ[b]);
        zero += r == 0;
      }
      CHECK(pkv_bm_free_blocks(m) == zero);
      if (!live.empty()) {
        std::vector<int32_t> seqs(live.begin(), live.end());
        std::vector<int32_t> tab(seqs.size() * MB), lens(seqs.size());
        CHECK(pkv_bm_tables(m, seqs.data(), (int32_t)seqs.size(), tab.data(), MB, -1, lens.data()) == PKV_OK);
      }
      int64_t used = -1, filled = -1, nlive = -1, held = -1;
      CHECK(pkv_bm_usage(m, &used, &filled, &nlive, &held) == PKV_OK);
      CHECK(used == NB - zero && nlive == (int64_t)live.size() && filled <= used * B);
    }
    pkv_bm_destroy(m);
  }
  printf("block manager sanitizer run: %d seeds ok\n", seeds);
  return 0;
}
