// Internal layout of the host block pool, shared by the pool and the prefix
// indexes (not part of the ABI).  Host memory only; no HIP calls.
#pragma once

#include <array>
#include <cstdint>
#include <memory>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

namespace pa {

using Hash = std::array<uint8_t, 32>;

struct Seq {
  std::vector<int32_t> table;  // GPU block ids, or host block ids when swapped
  int64_t fill = 0;
  bool swapped = false;
  // Prefix tracking: set when every token id of the sequence is known (created
  // through a prefix index and appended with token ids only).
  bool tracked = false;
  std::vector<int32_t> pending;  // token ids of the partly filled last block
  Hash chain{};                  // chain hash of the last full block (zeros before it)
  std::string key;               // salt and extra bytes of the request
  int32_t node = -1;             // radix position: node and blocks matched in it
  int32_t node_off = 0;
};

// FIFO of free block ids over [0, n)
struct Ring {
  std::vector<int32_t> buf;
  int64_t head = 0, count = 0;
  void init(int32_t n, const int32_t* order) {
    buf.resize(n);
    for (int32_t i = 0; i < n; ++i) buf[i] = order ? order[i] : i;
    head = 0;
    count = n;
  }
  int32_t pop() {
    const int32_t b = buf[head];
    head = (head + 1) % static_cast<int64_t>(buf.size());
    --count;
    return b;
  }
  void push(int32_t b) {
    buf[(head + count) % static_cast<int64_t>(buf.size())] = b;
    ++count;
  }
  int32_t at(int64_t i) const { return buf[(head + i) % static_cast<int64_t>(buf.size())]; }
};

struct Pool;

// A prefix index holds one reference on every block it indexes.  The pool
// reports when such a block loses its last sequence reference (idle) or gains
// one again (busy), and asks the index to evict idle blocks when the free
// list is short.
struct PrefixIndex {
  virtual ~PrefixIndex() = default;
  virtual int kind() const = 0;
  // Blocks that eviction could free now, not counting blocks in `keep` (and,
  // for the tree, the nodes that hold them).
  virtual int64_t evictable(const Pool& p, const std::vector<int32_t>& keep) const = 0;
  virtual void evict(Pool& p, int64_t k) = 0;  // free >= k blocks (k <= evictable)
  virtual void on_idle(Pool& p, int32_t b) = 0;
  virtual void on_busy(Pool& p, int32_t b) = 0;
  // Pure lookup of the full blocks of tokens[0..n) that end before the last
  // token: matched blocks in logical order, plus an opaque position.
  struct Pos {
    Hash chain{};
    int32_t node = -1, off = 0;
  };
  virtual void lookup(const Pool& p, const std::string& key, const int32_t* tokens, int64_t n,
                      std::vector<int32_t>& hits, Pos& pos) const = 0;
  // Commit a lookup for sequence `id` (stats, recency, tracking position).
  virtual void commit(Pool& p, int64_t id, Seq& s, const std::vector<int32_t>& hits,
                      const Pos& pos, int64_t queried) = 0;
  // Block b (logical index `depth`) of tracked sequence `id` has just been
  // filled with tokens[0..bs).
  virtual void add_full_block(Pool& p, int64_t id, Seq& s, int32_t b, int64_t depth,
                              const int32_t* tokens) = 0;
  virtual void on_fork(Pool&, int64_t /*child*/, Seq& /*child*/) {}
  virtual void untrack(Pool&, int64_t /*id*/, Seq& /*s*/) {}
  virtual int64_t indexed() const = 0;
  virtual int64_t nodes() const { return 0; }
  int64_t hits = 0, queried = 0, evicted = 0;
};

std::unique_ptr<PrefixIndex> make_hash_index(int32_t num_blocks);
std::unique_ptr<PrefixIndex> make_radix_index(int32_t num_blocks);

struct Pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  Ring gpu;                    // free GPU blocks
  std::vector<int32_t> ref;    // all references (sequences + index)
  std::vector<uint8_t> idx;    // 1 if a prefix index holds the block
  std::unordered_map<int64_t, Seq> seqs;
  int64_t copies = 0;
  int64_t tokens = 0;
  int64_t shared = 0;          // blocks with more than one sequence reference
  // host blocks for swapped sequences
  Ring host;
  std::vector<int32_t> host_ref;
  int64_t host_used = 0;
  int64_t swapped = 0;
  std::unique_ptr<PrefixIndex> index;
  int64_t tick = 0;            // advanced by every public operation

  int32_t seq_refs(int32_t b) const { return ref[b] - idx[b]; }
  int32_t alloc() {
    const int32_t b = gpu.pop();
    ref[b] = 1;
    idx[b] = 0;
    return b;
  }
  void retain(int32_t b) {
    ++ref[b];
    const int32_t s = seq_refs(b);
    if (s == 2) ++shared;
    if (s == 1 && idx[b]) index->on_busy(*this, b);
  }
  void release(int32_t b) {
    if (seq_refs(b) == 2) --shared;
    if (--ref[b] == 0) {
      gpu.push(b);
    } else if (idx[b] && seq_refs(b) == 0) {
      index->on_idle(*this, b);
    }
  }
  void index_hold(int32_t b) {  // the index takes a reference on a block
    idx[b] = 1;
    ++ref[b];
  }
  void index_drop(int32_t b) {  // eviction: the index gives it up
    idx[b] = 0;
    if (--ref[b] == 0) gpu.push(b);
  }
  // true if `need` blocks can be allocated now, evicting idle indexed blocks
  // if the free list alone is short
  bool ensure(int64_t need) {
    if (need <= gpu.count) return true;
    if (!index || gpu.count + index->evictable(*this, {}) < need) return false;
    index->evict(*this, need - gpu.count);
    return need <= gpu.count;
  }
  // a tracked sequence stops feeding the index
  void untrack(int64_t id, Seq& s) {
    if (s.tracked && index) index->untrack(*this, id, s);
    s.tracked = false;
    s.pending.clear();
  }
  void host_release(int32_t h) {
    if (--host_ref[h] == 0) {
      host.push(h);
      --host_used;
    }
  }
};

// Blocks that appending k tokens to `s` takes, when the refcount of its last
// block is `last_ref`.
inline int64_t blocks_needed(const Seq& s, int64_t k, int32_t bs, int32_t last_ref) {
  if (k <= 0) return 0;
  const int64_t n = s.fill;
  // positions n .. n+k-1 that start a block
  int64_t need = (n + k + bs - 1) / bs - (n + bs - 1) / bs;
  if (n % bs != 0 && last_ref > 1) need += 1;
  return need;
}

}  // namespace pa

struct pa_pool : pa::Pool {};
