// Random sequences of the host API (block pool, forks, appends, beam steps,
// swap, both prefix indexes, dense tables, decode order, cascade plan), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_fuzz.py.  After every operation the pool's block accounting
// is checked against what the public queries report:
//   free + used = pool size; the free list holds each block with refcount 0
//   exactly once; every block's refcount = references from the tables of
//   GPU-resident sequences + one per block the prefix index holds;
//   host free + host used = host pool size.
// Status codes are checked against the ones each call documents.  Prints a
// coverage line (how often the failure paths and the caches were reached)
// and "ok".
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "../include/pa.h"

namespace {

int g_iter;
unsigned g_seed;

#define CHECK(c)                                                                        \
  do {                                                                                  \
    if (!(c)) {                                                                         \
      std::fprintf(stderr, "FAIL %s:%d %s (seed %u, op %d)\n", __FILE__, __LINE__, #c, \
                   g_seed, g_iter);                                                     \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

struct Coverage {
  long no_blocks = 0, cow_pairs = 0, cached_hits = 0, evicted = 0, swaps = 0,
       beam_steps = 0, plans_with_groups = 0;
};

void check_accounting(pa_pool* p, int nb, int nhost, const std::set<int64_t>& live,
                      int prefix_kind) {
  int64_t st[5];
  CHECK(pa_pool_stats(p, st) == PA_OK);
  CHECK(st[0] + st[1] == nb);
  std::vector<int32_t> fl(nb + 1);
  int nf = 0;
  CHECK(pa_pool_free_list(p, fl.data(), nb + 1, &nf) == PA_OK);
  CHECK(nf == st[0]);
  std::vector<int> is_free(nb, 0);
  for (int i = 0; i < nf; ++i) {
    CHECK(fl[i] >= 0 && fl[i] < nb);
    CHECK(!is_free[fl[i]]);
    is_free[fl[i]] = 1;
  }
  std::vector<int64_t> refs(nb, 0);
  for (int64_t s : live) {
    const int sw = pa_seq_is_swapped(p, s);
    CHECK(sw == 0 || sw == 1);
    if (sw == 1) continue;
    int n = 0, t = 0;
    pa_status r = pa_seq_block_table(p, s, nullptr, 0, &n, &t);
    CHECK(r == PA_OK || r == PA_ERR_INVALID);
    std::vector<int32_t> tab(n + 1);
    CHECK(pa_seq_block_table(p, s, tab.data(), n + 1, &n, &t) == PA_OK);
    for (int i = 0; i < n; ++i) {
      CHECK(tab[i] >= 0 && tab[i] < nb);
      refs[tab[i]]++;
    }
  }
  int64_t indexed = 0;
  if (prefix_kind) {
    int64_t ps[6];
    CHECK(pa_prefix_stats(p, ps) == PA_OK);
    indexed = ps[0];
  }
  int64_t index_refs = 0, used = 0;
  for (int b = 0; b < nb; ++b) {
    const int rc = pa_pool_refcount(p, b);
    CHECK(rc >= refs[b]);
    CHECK((rc == 0) == (is_free[b] == 1));
    index_refs += rc - refs[b];
    used += rc > 0;
  }
  CHECK(used == st[1]);
  CHECK(index_refs == indexed);
  CHECK(pa_pool_refcount(p, -1) == -1 && pa_pool_refcount(p, nb) == -1);
  if (nhost) {
    int64_t hs[3];
    CHECK(pa_pool_host_stats(p, hs) == PA_OK);
    CHECK(hs[0] + hs[1] == nhost);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int runs = argc > 1 ? std::atoi(argv[1]) : 200;
  const int ops = argc > 2 ? std::atoi(argv[2]) : 400;
  Coverage cov;
  for (int run = 0; run < runs; ++run) {
    g_seed = 1000u + static_cast<unsigned>(run);
    std::mt19937 rng(g_seed);
    auto R = [&](int n) { return static_cast<int>(rng() % static_cast<unsigned>(n)); };
    const int bs = R(2) ? 16 : 32;
    const int nb = R(2) ? 4 + R(28) : 8 + R(120);  // small pools run out often
    std::vector<int32_t> order(nb);
    for (int i = 0; i < nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    pa_pool* p = nullptr;
    CHECK(pa_pool_create(nb, bs, R(2) ? order.data() : nullptr, &p) == PA_OK);
    const int kind = R(3);  // 0: no index, PA_PREFIX_HASH, PA_PREFIX_RADIX
    if (kind) CHECK(pa_pool_enable_prefix_cache(p, kind) == PA_OK);
    const int nhost = R(3) ? 4 + R(80) : 0;
    if (nhost) CHECK(pa_pool_set_host_blocks(p, nhost) == PA_OK);
    const int vocab = 1 + R(4);  // few token ids: prompts share prefixes
    std::set<int64_t> live;
    int64_t next_id = 1;
    for (g_iter = 0; g_iter < ops; ++g_iter) {
      const std::vector<int64_t> lv(live.begin(), live.end());
      auto pick = [&]() { return lv[R(static_cast<int>(lv.size()))]; };
      const int op = lv.empty() ? 0 : R(11);
      if (op == 0) {  // new sequence, from a prompt when an index is attached
        const int64_t id = next_id++;
        if (kind && R(2)) {
          const int n = 1 + R(3 * bs + 5);
          std::vector<int32_t> toks(n);
          for (auto& t : toks) t = R(vocab);
          const uint8_t salt[3] = {static_cast<uint8_t>(R(2)), 1, 2};
          int cached = -1;
          std::vector<int64_t> slots(n);
          const pa_status s = pa_seq_create_cached(p, id, toks.data(), n, salt,
                                                   R(2) ? 1 + R(3) : 0, nullptr, 0, &cached,
                                                   slots.data());
          CHECK(s == PA_OK || s == PA_ERR_NO_BLOCKS);
          if (s == PA_ERR_NO_BLOCKS) cov.no_blocks++;
          if (s == PA_OK) {
            CHECK(cached >= 0 && cached < n && cached % bs == 0);
            cov.cached_hits += cached > 0;
            for (int i = 0; i < n - cached; ++i)
              CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * bs);
            live.insert(id);
          }
        } else {
          CHECK(pa_seq_create(p, id) == PA_OK);
          live.insert(id);
        }
      } else if (op == 1) {  // fork
        const int64_t par = pick(), id = next_id++;
        const pa_status s = pa_seq_fork(p, par, id);
        CHECK(s == PA_OK || (s == PA_ERR_INVALID && pa_seq_is_swapped(p, par) == 1));
        if (s == PA_OK) live.insert(id);
      } else if (op == 2) {  // append to one sequence
        const int64_t s0 = pick();
        const int nt = 1 + R(R(2) ? 2 * bs : 3);
        std::vector<int64_t> slots(nt);
        int32_t pairs[2];
        int np = -1;
        const pa_status s = pa_seq_append(p, s0, nt, slots.data(), pairs, &np);
        CHECK(s == PA_OK || s == PA_ERR_NO_BLOCKS ||
              (s == PA_ERR_INVALID && pa_seq_is_swapped(p, s0) == 1));
        if (s == PA_ERR_NO_BLOCKS) cov.no_blocks++;
        if (s == PA_OK) {
          CHECK(np == 0 || np == 1);
          if (np) {
            cov.cow_pairs++;
            CHECK(pairs[0] != pairs[1] && pairs[0] >= 0 && pairs[0] < nb && pairs[1] >= 0 &&
                  pairs[1] < nb);
          }
          for (int i = 0; i < nt; ++i) CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * bs);
        }
      } else if (op == 3) {  // batch append of distinct ids, with token ids or without
        std::vector<int64_t> ids = lv;
        std::shuffle(ids.begin(), ids.end(), rng);
        ids.resize(1 + R(static_cast<int>(ids.size())));
        const int n = static_cast<int>(ids.size()), te = 1 + R(3);
        std::vector<int64_t> slots(static_cast<size_t>(n) * te);
        std::vector<int32_t> pairs(2 * n), toks(static_cast<size_t>(n) * te);
        for (auto& t : toks) t = R(vocab);
        int np = -1;
        const pa_status s =
            kind && R(2) ? pa_seq_append_tokens(p, ids.data(), n, toks.data(), te, slots.data(),
                                                pairs.data(), &np)
                         : pa_seq_append_batch(p, ids.data(), n, te, slots.data(), pairs.data(),
                                               &np);
        CHECK(s == PA_OK || s == PA_ERR_NO_BLOCKS || s == PA_ERR_INVALID);  // INVALID: swapped
        if (s == PA_ERR_NO_BLOCKS) cov.no_blocks++;
        if (s == PA_OK) CHECK(np >= 0 && np <= n);
      } else if (op == 4) {  // free
        const int64_t s0 = pick();
        CHECK(pa_seq_free(p, s0) == PA_OK);
        live.erase(s0);
        CHECK(pa_seq_is_swapped(p, s0) == -1);
      } else if (op == 5) {  // beam step over GPU-resident sequences
        std::vector<int64_t> old;
        for (int64_t s : lv)
          if (pa_seq_is_swapped(p, s) == 0 && R(2)) old.push_back(s);
        if (old.empty()) continue;
        const int n_new = R(4);
        std::vector<int64_t> par(n_new), nw(n_new), slots(n_new + 1);
        std::vector<int32_t> pairs(2 * n_new + 2);
        for (int j = 0; j < n_new; ++j) {
          par[j] = old[R(static_cast<int>(old.size()))];
          nw[j] = R(3) ? next_id++ : old[R(static_cast<int>(old.size()))];  // ids may be reused
        }
        int np = -1;
        const pa_status s =
            pa_seq_beam_step(p, old.data(), static_cast<int>(old.size()), par.data(), nw.data(),
                             n_new, nullptr, slots.data(), pairs.data(), &np);
        CHECK(s == PA_OK || s == PA_ERR_NO_BLOCKS || s == PA_ERR_INVALID);  // INVALID: repeats
        if (s == PA_ERR_NO_BLOCKS) cov.no_blocks++;
        if (s == PA_OK || s == PA_ERR_NO_BLOCKS) {  // the fork-and-retire part happened
          cov.beam_steps += s == PA_OK;
          for (int64_t o : old) live.erase(o);
          for (int64_t x : nw) live.insert(x);
        }
      } else if (op == 6 && nhost) {  // swap out or in
        std::vector<int64_t> ids;
        for (int64_t s : lv)
          if (R(3) == 0) ids.push_back(s);
        if (ids.empty()) continue;
        const int n = static_cast<int>(ids.size()), cap = nb + nhost;
        std::vector<int32_t> pairs(2 * cap);
        int np = -1;
        const pa_status s = R(2) ? pa_seq_swap_out(p, ids.data(), n, pairs.data(), cap, &np)
                                 : pa_seq_swap_in(p, ids.data(), n, pairs.data(), cap, &np);
        CHECK(s == PA_OK || s == PA_ERR_NO_BLOCKS || s == PA_ERR_INVALID);  // INVALID: state
        cov.swaps += s == PA_OK;
      } else if (op == 7) {  // dense tables, decode order and cascade plan
        std::vector<int64_t> ids;
        for (int64_t s : lv)
          if (pa_seq_is_swapped(p, s) == 0) ids.push_back(s);
        if (ids.empty()) continue;
        const int n = static_cast<int>(ids.size()), maxb = 1 + R(12);
        std::vector<int32_t> tab(static_cast<size_t>(n) * maxb), lens(n), ord(n);
        const pa_status s = pa_pool_block_tables(p, ids.data(), n, tab.data(), maxb, lens.data());
        CHECK(s == PA_OK || s == PA_ERR_INVALID);  // INVALID: a table longer than maxb
        if (s != PA_OK) continue;
        CHECK(pa_decode_order(tab.data(), maxb, lens.data(), n, ord.data()) == PA_OK);
        std::vector<int> seen(n, 0);
        for (int i = 0; i < n; ++i) {
          CHECK(ord[i] >= 0 && ord[i] < n && !seen[ord[i]]);
          seen[ord[i]] = 1;
        }
        std::vector<int32_t> pre(n), groups(3 * n), members(n);
        int ng = 0, mp = 0, mm = 0, mr = 0;
        const int G = 1 << R(5);
        CHECK(pa_cascade_plan(tab.data(), maxb, lens.data(), n, bs, 8 * G, 8, R(2) ? 32 : 0,
                              pre.data(), groups.data(), members.data(), &ng, &mp, &mm,
                              &mr) == PA_OK);
        CHECK(ng >= 0 && ng <= n && mm * G <= 32);
        cov.plans_with_groups += ng > 0;
        int maxL = 0;
        for (int gi = 0; gi < ng; ++gi) {
          const int first = groups[3 * gi], cnt = groups[3 * gi + 1], L = groups[3 * gi + 2];
          CHECK(first >= 0 && cnt >= 1 && first + cnt <= n && L > 0 && L % 32 == 0);
          maxL = std::max(maxL, L);
          const int32_t* t0 = tab.data() + static_cast<size_t>(members[first]) * maxb;
          for (int k = 0; k < cnt; ++k) {
            const int m = members[first + k];
            CHECK(m >= 0 && m < n && pre[m] == L && lens[m] >= L);
            const int32_t* tm = tab.data() + static_cast<size_t>(m) * maxb;
            for (int b = 0; b < (L + bs - 1) / bs; ++b) CHECK(tm[b] == t0[b]);
          }
        }
        CHECK(mp == maxL);
        int rest = 0;
        for (int i = 0; i < n; ++i) rest = std::max(rest, lens[i] - pre[i]);
        CHECK(mr == rest);
      } else if (op == 8) {  // documented error statuses leave the pool as it was
        CHECK(pa_seq_create(p, pick()) == PA_ERR_INVALID);
        CHECK(pa_seq_free(p, -12345) == PA_ERR_UNKNOWN_SEQ);
        int n = 0, t = 0;
        CHECK(pa_seq_block_table(p, -12345, nullptr, 0, &n, &t) == PA_ERR_UNKNOWN_SEQ);
        const int64_t twice[2] = {lv[0], lv[0]};
        int64_t sl[4];
        int32_t pr[4];
        int np = 0;
        CHECK(pa_seq_append_batch(p, twice, 2, 1, sl, pr, &np) == PA_ERR_INVALID);
      } else if (op == 9) {  // free about half
        for (int64_t s : lv)
          if (R(2)) {
            CHECK(pa_seq_free(p, s) == PA_OK);
            live.erase(s);
          }
      } else if (op == 10) {
        int64_t ps[6];
        CHECK(pa_prefix_stats(p, ps) == PA_OK);
        if (!kind)
          for (int i = 0; i < 6; ++i) CHECK(ps[i] == 0);
      }
      check_accounting(p, nb, nhost, live, kind);
    }
    if (kind) {
      int64_t ps[6];
      CHECK(pa_prefix_stats(p, ps) == PA_OK);
      cov.evicted += ps[4];
    }
    for (int64_t s : live) CHECK(pa_seq_free(p, s) == PA_OK);
    int64_t st[5];
    CHECK(pa_pool_stats(p, st) == PA_OK);
    if (!kind) CHECK(st[0] == nb);  // an index keeps its blocks
    pa_pool_destroy(p);
  }
  std::printf("coverage no_blocks=%ld cow_pairs=%ld cached_hits=%ld evicted=%ld swaps=%ld "
              "beam_steps=%ld plans_with_groups=%ld\n",
              cov.no_blocks, cov.cow_pairs, cov.cached_hits, cov.evicted, cov.swaps,
              cov.beam_steps, cov.plans_with_groups);
  std::printf("ok %d runs\n", runs);
  return 0;
}
