// Host-side KV block pool: per-sequence block tables, refcounts, fork / append /
// free and copy-on-write decisions (vLLM encyclopedia entry, tonho.wtf, section
// "como funciona"), and swapping whole sequences to host blocks and back
// (same entry, "a ideia" and "como funciona": swap to CPU RAM, eviction all or
// nothing per sequence).  Host memory only; no HIP calls.
//
// Each free list is a ring buffer holding each free block id once (FIFO: take
// from the front, return to the back).  Sequences live in a hash map keyed by
// the caller's 64-bit id.  Every operation is O(tokens + blocks touched).
// Prefix indexes (chain hashing, radix tree) live in pa_prefix.cpp and attach
// to the pool through the hooks in pa_pool_impl.h.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_pool_impl.h"

using namespace pa;

namespace {

void append_one(pa_pool* p, Seq& s, int64_t k, int64_t* slots, int32_t* pair, int* npairs) {
  const int32_t bs = p->block_size;
  for (int64_t j = 0; j < k; ++j) {
    const int64_t n = s.fill;
    if (n % bs == 0) {
      s.table.push_back(p->alloc());
    } else if (j == 0 && p->seq_refs(s.table.back()) > 1) {
      const int32_t old = s.table.back();
      const int32_t nb = p->alloc();
      pair[0] = old;
      pair[1] = nb;
      ++*npairs;
      ++p->copies;
      p->release(old);
      s.table.back() = nb;
    }
    slots[j] = static_cast<int64_t>(s.table.back()) * bs + n % bs;
    s.fill = n + 1;
  }
  p->tokens += k;
}

}  // namespace

PA_EXPORT pa_status pa_pool_create(int num_blocks, int block_size, const int32_t* free_order,
                                   pa_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID;
  *out = nullptr;
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return PA_ERR_INVALID;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign(num_blocks, 0);
  p->idx.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return PA_ERR_INVALID;
      }
      seen[b] = 1;
    }
  }
  p->gpu.init(num_blocks, free_order);
  *out = p;
  return PA_OK;
}

PA_EXPORT void pa_pool_destroy(pa_pool* pool) { delete pool; }

PA_EXPORT pa_status pa_seq_create(pa_pool* p, int64_t seq_id) {
  if (!p) return PA_ERR_INVALID;
  if (p->seqs.count(seq_id)) return PA_ERR_INVALID;
  p->seqs.emplace(seq_id, Seq());
  return PA_OK;
}

PA_EXPORT pa_status pa_seq_fork(pa_pool* p, int64_t parent, int64_t child) {
  if (!p) return PA_ERR_INVALID;
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (p->seqs.count(child) || it->second.swapped) return PA_ERR_INVALID;
  Seq c = it->second;  // copy before emplace (rehash may move it)
  for (int32_t b : c.table) p->retain(b);
  p->tokens += c.fill;
  Seq& cs = p->seqs.emplace(child, std::move(c)).first->second;
  if (cs.tracked && p->index) p->index->on_fork(*p, child, cs);
  return PA_OK;
}

namespace pa {

// Appends tokens_each positions to each sequence.  tokens (may be null) holds
// their token ids [n][tokens_each]: a tracked sequence then feeds every block
// it fills to the prefix index; without token ids a sequence stops being
// tracked.
pa_status append_batch_impl(pa_pool* p, const int64_t* seqs, int n, int tokens_each,
                            const int32_t* tokens, int64_t* slots_out, int32_t* pairs_out,
                            int* num_pairs_out) {
  if (!p || n < 0 || tokens_each < 0) return PA_ERR_INVALID;
  if (n > 0 && !seqs) return PA_ERR_INVALID;
  if (n > 0 && tokens_each > 0 && (!slots_out || !pairs_out)) return PA_ERR_INVALID;
  if (num_pairs_out) *num_pairs_out = 0;
  ++p->tick;
  // resolve ids, reject duplicates
  std::vector<Seq*> ss(n);
  for (int i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    ss[i] = &it->second;
  }
  for (int i = 0; i < n; ++i)
    if (ss[i]->swapped) return PA_ERR_INVALID;
  {
    std::vector<int64_t> ids(seqs, seqs + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) return PA_ERR_INVALID;
  }
  if (tokens_each == 0 || n == 0) return PA_OK;
  // dry run: blocks the whole batch takes, tracking refcount drops of copied blocks
  const int32_t bs = p->block_size;
  std::unordered_map<int32_t, int32_t> overlay;
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const Seq& s = *ss[i];
    int32_t last_ref = 0;
    int32_t last = -1;
    if (!s.table.empty()) {
      last = s.table.back();
      auto o = overlay.find(last);
      last_ref = (o == overlay.end()) ? p->seq_refs(last) : o->second;
    }
    need += blocks_needed(s, tokens_each, bs, last_ref);
    if (s.fill % bs != 0 && last_ref > 1) overlay[last] = last_ref - 1;
  }
  if (!p->ensure(need)) return PA_ERR_NO_BLOCKS;
  int np = 0;
  for (int i = 0; i < n; ++i) {
    int got = 0;
    Seq& s = *ss[i];
    int64_t* sl = slots_out + static_cast<int64_t>(i) * tokens_each;
    append_one(p, s, tokens_each, sl, pairs_out + 2 * np, &got);
    np += got;
    if (!tokens) {
      p->untrack(seqs[i], s);
      continue;
    }
    if (!s.tracked) continue;
    const int32_t* tk = tokens + static_cast<int64_t>(i) * tokens_each;
    const int64_t first = s.fill - tokens_each;
    for (int j = 0; j < tokens_each && s.tracked; ++j) {
      s.pending.push_back(tk[j]);
      if (static_cast<int32_t>(s.pending.size()) == bs) {
        p->index->add_full_block(*p, seqs[i], s, static_cast<int32_t>(sl[j] / bs),
                                 (first + j) / bs, s.pending.data());
        s.pending.clear();
      }
    }
  }
  if (num_pairs_out) *num_pairs_out = np;
  return PA_OK;
}

}  // namespace pa

PA_EXPORT pa_status pa_seq_append_batch(pa_pool* p, const int64_t* seqs, int n, int tokens_each,
                                        int64_t* slots_out, int32_t* pairs_out,
                                        int* num_pairs_out) {
  return append_batch_impl(p, seqs, n, tokens_each, nullptr, slots_out, pairs_out,
                           num_pairs_out);
}

PA_EXPORT pa_status pa_seq_append_tokens(pa_pool* p, const int64_t* seqs, int n,
                                         const int32_t* tokens, int tokens_each,
                                         int64_t* slots_out, int32_t* pairs_out,
                                         int* num_pairs_out) {
  if (n > 0 && tokens_each > 0 && !tokens) return PA_ERR_INVALID;
  return append_batch_impl(p, seqs, n, tokens_each, tokens, slots_out, pairs_out,
                           num_pairs_out);
}

PA_EXPORT pa_status pa_seq_append(pa_pool* p, int64_t seq, int num_tokens, int64_t* slots_out,
                                  int32_t* pairs_out, int* num_pairs_out) {
  return pa_seq_append_batch(p, &seq, 1, num_tokens, slots_out, pairs_out, num_pairs_out);
}

namespace {

void free_impl(pa_pool* p, std::unordered_map<int64_t, Seq>::iterator it) {
  p->untrack(it->first, it->second);
  if (it->second.swapped) {
    for (int32_t h : it->second.table) p->host_release(h);
    --p->swapped;
  } else {
    for (int32_t b : it->second.table) p->release(b);
  }
  p->tokens -= it->second.fill;
  p->seqs.erase(it);
}

}  // namespace

PA_EXPORT pa_status pa_seq_free(pa_pool* p, int64_t seq) {
  if (!p) return PA_ERR_INVALID;
  ++p->tick;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  free_impl(p, it);
  return PA_OK;
}

PA_EXPORT pa_status pa_seq_beam_step(pa_pool* p, const int64_t* old_beams, int n_old,
                                     const int64_t* parents, const int64_t* new_beams, int n_new,
                                     const int32_t* tokens, int64_t* slots_out,
                                     int32_t* pairs_out, int* num_pairs_out) {
  if (!p || n_old < 0 || n_new < 0) return PA_ERR_INVALID;
  if ((n_old > 0 && !old_beams) ||
      (n_new > 0 && (!parents || !new_beams || !slots_out || !pairs_out)))
    return PA_ERR_INVALID;
  if (num_pairs_out) *num_pairs_out = 0;
  std::vector<std::unordered_map<int64_t, Seq>::iterator> olds(n_old);
  for (int i = 0; i < n_old; ++i) {
    olds[i] = p->seqs.find(old_beams[i]);
    if (olds[i] == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  }
  std::unordered_map<int64_t, int> is_old;
  for (int i = 0; i < n_old; ++i) {
    if (olds[i]->second.swapped) return PA_ERR_INVALID;
    if (!is_old.emplace(old_beams[i], i).second) return PA_ERR_INVALID;
  }
  {
    std::vector<int64_t> ids(new_beams, new_beams + n_new);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) return PA_ERR_INVALID;
  }
  for (int j = 0; j < n_new; ++j) {
    if (!is_old.count(parents[j])) return PA_ERR_INVALID;
    if (p->seqs.count(new_beams[j]) && !is_old.count(new_beams[j])) return PA_ERR_INVALID;
  }
  ++p->tick;
  if (p->index) {
    // 1. the new beams map their parents' blocks (before any old beam goes)
    std::vector<Seq> kids;
    kids.reserve(n_new);
    for (int j = 0; j < n_new; ++j) {
      kids.push_back(olds[is_old[parents[j]]]->second);
      for (int32_t b : kids.back().table) p->retain(b);
      p->tokens += kids.back().fill;
    }
    // 2. the old beams retire
    for (int i = 0; i < n_old; ++i) free_impl(p, p->seqs.find(old_beams[i]));
    // 3. the new beams take their ids
    for (int j = 0; j < n_new; ++j) {
      Seq& cs = p->seqs.emplace(new_beams[j], std::move(kids[j])).first->second;
      if (cs.tracked && p->index) p->index->on_fork(*p, new_beams[j], cs);
    }
  } else {
    // Without a prefix index, the same result with less work: the first
    // child of an old beam takes over its record and its references (no copy
    // and no retain / release pair), further children copy it, and records
    // of childless beams are reused for those copies.
    std::vector<int> nkids(n_old, 0), first_kid(n_old, -1), par(n_new);
    for (int j = 0; j < n_new; ++j) {
      const int i = is_old[parents[j]];
      par[j] = i;
      if (nkids[i]++ == 0) first_kid[i] = j;
    }
    // 1. the further children's references, all before any release (as when
    //    every child retains first), so no block shared with a childless
    //    beam reaches zero early
    for (int i = 0; i < n_old; ++i) {
      if (nkids[i] < 2) continue;
      const Seq& s = olds[i]->second;
      for (int32_t b : s.table)
        for (int k = 1; k < nkids[i]; ++k) p->retain(b);
      p->tokens += static_cast<int64_t>(nkids[i] - 1) * s.fill;
    }
    // 2. the old beams leave the map; childless ones release their blocks in
    //    beam order, then in table order, so blocks reach the free list in
    //    the same order as when every old beam retires after the retains
    std::vector<std::unordered_map<int64_t, Seq>::node_type> nodes(n_old);
    for (int i = 0; i < n_old; ++i) nodes[i] = p->seqs.extract(olds[i]);
    std::vector<int> spare;
    for (int i = 0; i < n_old; ++i) {
      if (nkids[i] > 0) continue;
      Seq& s = nodes[i].mapped();
      for (int32_t b : s.table) p->release(b);
      p->tokens -= s.fill;
      spare.push_back(i);
    }
    // 3. the new beams take their ids: further children first (their
    //    parents' records are still out of the map), then first children
    size_t next = 0;
    for (int j = 0; j < n_new; ++j) {
      const int i = par[j];
      if (first_kid[i] == j) continue;
      const Seq& src = nodes[i].mapped();
      if (next < spare.size()) {
        auto& nh = nodes[spare[next++]];
        nh.mapped() = src;
        nh.key() = new_beams[j];
        p->seqs.insert(std::move(nh));
      } else {
        p->seqs.emplace(new_beams[j], src);
      }
    }
    for (int i = 0; i < n_old; ++i) {
      if (first_kid[i] < 0) continue;
      nodes[i].key() = new_beams[first_kid[i]];
      p->seqs.insert(std::move(nodes[i]));
    }
  }
  // 4. one token each, copy-on-write in the order given
  return append_batch_impl(p, new_beams, n_new, n_new > 0 ? 1 : 0, tokens, slots_out, pairs_out,
                           num_pairs_out);
}

PA_EXPORT pa_status pa_seq_block_table(const pa_pool* p, int64_t seq, int32_t* out, int cap,
                                       int* num_blocks_out, int* num_tokens_out) {
  if (!p || cap < 0) return PA_ERR_INVALID;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const Seq& s = it->second;
  const int64_t nb = static_cast<int64_t>(s.table.size());
  if (num_blocks_out) *num_blocks_out = static_cast<int>(nb);
  if (num_tokens_out) *num_tokens_out = static_cast<int>(s.fill);
  if (nb > cap) return PA_ERR_INVALID;
  if (nb && !out) return PA_ERR_INVALID;
  if (nb) std::memcpy(out, s.table.data(), nb * sizeof(int32_t));
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_block_tables(const pa_pool* p, const int64_t* seqs, int n,
                                         int32_t* out, int maxb, int32_t* lens_out) {
  if (!p || n < 0 || maxb < 0) return PA_ERR_INVALID;
  if (n > 0 && (!seqs || !out || !lens_out)) return PA_ERR_INVALID;
  std::vector<const Seq*> ss(n);
  for (int i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PA_ERR_INVALID;
    if (static_cast<int64_t>(it->second.table.size()) > maxb) return PA_ERR_INVALID;
    ss[i] = &it->second;
  }
  for (int i = 0; i < n; ++i) {
    int32_t* row = out + static_cast<int64_t>(i) * maxb;
    const auto& t = ss[i]->table;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + maxb, -1);
    lens_out[i] = static_cast<int32_t>(ss[i]->fill);
  }
  return PA_OK;
}

PA_EXPORT int pa_pool_refcount(const pa_pool* p, int32_t block) {
  if (!p || block < 0 || block >= p->num_blocks) return -1;
  return p->ref[block];
}

PA_EXPORT pa_status pa_pool_free_list(const pa_pool* p, int32_t* out, int cap, int* n_out) {
  if (!p || cap < 0) return PA_ERR_INVALID;
  if (n_out) *n_out = static_cast<int>(p->gpu.count);
  if (p->gpu.count > cap) return PA_ERR_INVALID;
  if (p->gpu.count && !out) return PA_ERR_INVALID;
  for (int64_t i = 0; i < p->gpu.count; ++i) out[i] = p->gpu.at(i);
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_stats(const pa_pool* p, int64_t* stats_out) {
  if (!p || !stats_out) return PA_ERR_INVALID;
  int64_t used = 0;
  for (int32_t r : p->ref) used += r > 0;
  stats_out[0] = p->gpu.count;
  stats_out[1] = used;
  stats_out[2] = p->shared;
  stats_out[3] = p->tokens;
  stats_out[4] = p->copies;
  return PA_OK;
}

// Internal (not in the ABI): number of blocks currently held by more than one
// sequence, O(1).
extern "C" __attribute__((visibility("hidden"))) int64_t pa_pool_shared_blocks(const pa_pool* p) {
  return p ? p->shared : 0;
}

PA_EXPORT pa_status pa_pool_set_host_blocks(pa_pool* p, int num_host_blocks) {
  if (!p || num_host_blocks < 0) return PA_ERR_INVALID;
  if (p->swapped > 0) return PA_ERR_INVALID;
  p->host.init(num_host_blocks, nullptr);
  p->host_ref.assign(num_host_blocks, 0);
  p->host_used = 0;
  return PA_OK;
}

namespace {

// Resolve a batch of distinct ids whose swapped state is `want_swapped`.
pa_status resolve_batch(pa_pool* p, const int64_t* seqs, int n, bool want_swapped,
                        std::vector<Seq*>& out) {
  if (n < 0 || (n > 0 && !seqs)) return PA_ERR_INVALID;
  out.resize(n);
  for (int i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    out[i] = &it->second;
  }
  for (int i = 0; i < n; ++i)
    if (out[i]->swapped != want_swapped) return PA_ERR_INVALID;
  std::vector<int64_t> ids(seqs, seqs + n);
  std::sort(ids.begin(), ids.end());
  if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) return PA_ERR_INVALID;
  return PA_OK;
}

// Distinct block ids of the batch's tables in order of first appearance
// (sequence order, then logical order); `slot` maps an id to its index.
void distinct_blocks(const std::vector<Seq*>& ss, std::vector<int32_t>& uniq,
                     std::unordered_map<int32_t, int32_t>& slot) {
  for (const Seq* s : ss)
    for (int32_t b : s->table)
      if (slot.emplace(b, static_cast<int32_t>(uniq.size())).second) uniq.push_back(b);
}

}  // namespace

PA_EXPORT pa_status pa_seq_swap_out(pa_pool* p, const int64_t* seqs, int n, int32_t* pairs_out,
                                    int cap, int* num_pairs_out) {
  if (!p || cap < 0) return PA_ERR_INVALID;
  ++p->tick;
  if (num_pairs_out) *num_pairs_out = 0;
  std::vector<Seq*> ss;
  pa_status st = resolve_batch(p, seqs, n, false, ss);
  if (st != PA_OK) return st;
  std::vector<int32_t> uniq;
  std::unordered_map<int32_t, int32_t> slot;
  distinct_blocks(ss, uniq, slot);
  const int64_t k = static_cast<int64_t>(uniq.size());
  if (k > cap || (k > 0 && !pairs_out)) return PA_ERR_INVALID;
  if (k > p->host.count) return PA_ERR_NO_BLOCKS;
  std::vector<int32_t> hb(k);
  for (int64_t i = 0; i < k; ++i) {
    hb[i] = p->host.pop();
    pairs_out[2 * i] = uniq[i];
    pairs_out[2 * i + 1] = hb[i];
  }
  p->host_used += k;
  for (int i = 0; i < n; ++i) p->untrack(seqs[i], *ss[i]);
  for (Seq* s : ss) {
    for (int32_t& b : s->table) {
      const int32_t h = hb[slot[b]];
      ++p->host_ref[h];
      p->release(b);
      b = h;
    }
    s->swapped = true;
    ++p->swapped;
  }
  if (num_pairs_out) *num_pairs_out = static_cast<int>(k);
  return PA_OK;
}

PA_EXPORT pa_status pa_seq_swap_in(pa_pool* p, const int64_t* seqs, int n, int32_t* pairs_out,
                                   int cap, int* num_pairs_out) {
  if (!p || cap < 0) return PA_ERR_INVALID;
  ++p->tick;
  if (num_pairs_out) *num_pairs_out = 0;
  std::vector<Seq*> ss;
  pa_status st = resolve_batch(p, seqs, n, true, ss);
  if (st != PA_OK) return st;
  std::vector<int32_t> uniq;
  std::unordered_map<int32_t, int32_t> slot;
  distinct_blocks(ss, uniq, slot);
  const int64_t k = static_cast<int64_t>(uniq.size());
  if (k > cap || (k > 0 && !pairs_out)) return PA_ERR_INVALID;
  if (!p->ensure(k)) return PA_ERR_NO_BLOCKS;
  std::vector<int32_t> gb(k);
  std::vector<char> first(k, 1);
  for (int64_t i = 0; i < k; ++i) {
    gb[i] = p->alloc();
    pairs_out[2 * i] = uniq[i];
    pairs_out[2 * i + 1] = gb[i];
  }
  for (Seq* s : ss) {
    for (int32_t& h : s->table) {
      const int32_t j = slot[h];
      const int32_t g = gb[j];
      if (first[j]) {
        first[j] = 0;  // alloc() gave the first reference
      } else {
        p->retain(g);
      }
      p->host_release(h);
      h = g;
    }
    s->swapped = false;
    --p->swapped;
  }
  if (num_pairs_out) *num_pairs_out = static_cast<int>(k);
  return PA_OK;
}

PA_EXPORT int pa_seq_is_swapped(const pa_pool* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return -1;
  return it->second.swapped ? 1 : 0;
}

PA_EXPORT pa_status pa_pool_host_stats(const pa_pool* p, int64_t* stats_out) {
  if (!p || !stats_out) return PA_ERR_INVALID;
  stats_out[0] = p->host.count;
  stats_out[1] = p->host_used;
  stats_out[2] = p->swapped;
  return PA_OK;
}

PA_EXPORT pa_status pa_decode_order(const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int num_seqs,
                                    int32_t* order_out) {
  if (num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !order_out) return PA_ERR_INVALID;
  // group = sequences whose table starts with the same physical block (a fork
  // or a shared prefix always shares from the first block); an empty
  // sequence or one without a first block is a group of its own
  std::vector<int32_t> group(num_seqs), gmax;
  std::unordered_map<int32_t, int32_t> first;
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t b0 = block_tables[static_cast<size_t>(s) * max_blocks_per_seq];
    const int32_t len = context_lens[s];
    int32_t g;
    if (len > 0 && max_blocks_per_seq > 0 && b0 >= 0) {
      auto it = first.find(b0);
      if (it == first.end()) {
        g = static_cast<int32_t>(gmax.size());
        first.emplace(b0, g);
        gmax.push_back(len);
      } else {
        g = it->second;
        gmax[g] = std::max(gmax[g], len);
      }
    } else {
      g = static_cast<int32_t>(gmax.size());
      gmax.push_back(len);
    }
    group[s] = g;
  }
  for (int s = 0; s < num_seqs; ++s) order_out[s] = s;
  std::sort(order_out, order_out + num_seqs, [&](int32_t x, int32_t y) {
    const int32_t gx = group[x], gy = group[y];
    if (gmax[gx] != gmax[gy]) return gmax[gx] > gmax[gy];
    if (gx != gy) return gx < gy;
    if (context_lens[x] != context_lens[y]) return context_lens[x] > context_lens[y];
    return x < y;
  });
  return PA_OK;
}

PA_EXPORT pa_status pa_cascade_plan(const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int num_seqs, int block_size,
                                    int num_q_heads, int num_kv_heads, int min_prefix,
                                    int32_t* prefix_len_out, int32_t* groups_out,
                                    int32_t* members_out, int* num_groups_out,
                                    int* max_prefix_out, int* max_members_out,
                                    int* max_rest_out) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || !num_groups_out ||
      !max_prefix_out || !max_members_out || !max_rest_out)
    return PA_ERR_INVALID;
  *num_groups_out = 0;
  *max_prefix_out = 0;
  *max_members_out = 0;
  *max_rest_out = 0;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !prefix_len_out || !groups_out || !members_out)
    return PA_ERR_INVALID;
  for (int s = 0; s < num_seqs; ++s) prefix_len_out[s] = 0;
  // the longest context outside any group's prefix (updated below)
  auto rest = [&]() {
    int r = 0;
    for (int s = 0; s < num_seqs; ++s)
      r = std::max(r, std::max(context_lens[s], 0) - prefix_len_out[s]);
    *max_rest_out = r;
  };
  const int G = num_q_heads / num_kv_heads;
  const int cap = G <= 16 ? 32 / G : 0;  // sequences per 2 x 16 MFMA columns
  if (max_blocks_per_seq == 0 || cap == 0) {
    rest();
    return PA_OK;
  }
  // families: sequences whose tables start with the same physical block, in
  // order of first appearance, members in index order
  std::unordered_map<int32_t, int32_t> fam_of;
  std::vector<std::vector<int32_t>> fams;
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t b0 = block_tables[static_cast<size_t>(s) * max_blocks_per_seq];
    if (context_lens[s] <= 0 || b0 < 0) continue;
    auto it = fam_of.emplace(b0, static_cast<int32_t>(fams.size()));
    if (it.second) fams.emplace_back();
    fams[it.first->second].push_back(s);
  }
  int ng = 0, nm = 0;
  for (const auto& f : fams) {
    if (f.size() < 2) continue;
    int min_len = context_lens[f[0]];
    for (int32_t s : f) min_len = std::min(min_len, context_lens[s]);
    const int nb = std::min((min_len + block_size - 1) / block_size, max_blocks_per_seq);
    // the run of leading entries every member shares with the first: each
    // row against the first one, contiguously
    const int32_t* t0 = block_tables + static_cast<size_t>(f[0]) * max_blocks_per_seq;
    int common = nb;
    for (size_t i = 1; i < f.size() && common > 0; ++i) {
      const int32_t* ti = block_tables + static_cast<size_t>(f[i]) * max_blocks_per_seq;
      common = static_cast<int>(std::mismatch(t0, t0 + common, ti).first - t0);
    }
    int L = std::min(common * block_size, min_len) & ~31;
    if (L < std::max(min_prefix, 32)) continue;
    for (size_t i = 0; i < f.size(); i += cap) {
      const int cnt = static_cast<int>(std::min(f.size() - i, static_cast<size_t>(cap)));
      groups_out[3 * ng] = nm;
      groups_out[3 * ng + 1] = cnt;
      groups_out[3 * ng + 2] = L;
      for (int k = 0; k < cnt; ++k) {
        members_out[nm++] = f[i + k];
        prefix_len_out[f[i + k]] = L;
      }
      *max_members_out = std::max(*max_members_out, cnt);
      ++ng;
    }
    *max_prefix_out = std::max(*max_prefix_out, L);
  }
  *num_groups_out = ng;
  rest();
  return PA_OK;
}

PA_EXPORT size_t pa_kv_bytes_per_token(int num_layers, int num_kv_heads, int head_dim,
                                       int dtype) {
  size_t e;
  switch (dtype) {
    case PA_F32: e = 4; break;
    case PA_F16:
    case PA_BF16: e = 2; break;
    default: return 0;
  }
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0) return 0;
  return 2 * static_cast<size_t>(num_layers) * num_kv_heads * head_dim * e;
}

PA_EXPORT const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_UNKNOWN_SEQ: return "unknown sequence id";
    case PA_ERR_HIP: return "HIP launch or runtime error";
    case PA_ERR_TOO_LARGE: return "request exceeds the fixed no-allocation scratch";
    default: return "unknown status";
  }
}

PA_EXPORT int pa_abi_version(void) { return 5; }
