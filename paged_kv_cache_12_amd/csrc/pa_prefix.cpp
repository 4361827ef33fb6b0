// Automatic prefix reuse on top of the block pool: an index finds the blocks
// that already hold a request's prompt prefix, so only the rest is computed
// (aitalk.it "RadixAttention: un albero che non dimentica" and "Due strati,
// non due rivali"; "KV Cache Administration", sections "How RadixAttention
// Works", "How vLLM Implements Prefix Caching" and "Cache salting prevents
// cross-tenant reuse").  Two interchangeable indexes:
//
//  * chain hashing: a full block's key is SHA-256 over its parent block's key,
//    its token ids and the request's extra bytes (the tenant salt enters the
//    first block, so every later key differs per tenant); lookup walks the
//    prompt's blocks in order and stops at the first miss;
//  * a radix tree: a compressed trie over token ids at block granularity, one
//    root per (salt, extra); match walks the tree, insert splits a node where
//    a new request diverges, eviction removes least recently used leaves whose
//    blocks no sequence holds, so shared inner nodes outlive their leaves.
//
// Both hold one pool reference per indexed block: a cached block outlives the
// requests that wrote it and is evicted only when the free list is short.
// Host memory only; no HIP calls.
#include <immintrin.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <set>
#include <tuple>
#include <unordered_set>

#include "pa_pool_impl.h"

namespace pa {

// ---------------------------------------------------------------------------
// SHA-256 (FIPS 180-4).  kK is the standard's table of 64 round constants
// (section 4.2.2) and the initial hash value below is its section 5.3.3;
// both are data of the published algorithm, taken from the standard (the
// initial value is in the Sha256 constructor below).
// ---------------------------------------------------------------------------
namespace {

constexpr uint32_t kK[64] = {
    0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
    0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
    0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
    0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
    0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
    0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
    0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
    0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
    0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
    0xc67178f2};

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// One 64-byte block at a time, straight from the standard's definitions.
void compress_portable(uint32_t h[8], const uint8_t* m, size_t nblocks) {
  for (; nblocks; --nblocks, m += 64) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t(m[4 * t]) << 24) | (uint32_t(m[4 * t + 1]) << 16) |
             (uint32_t(m[4 * t + 2]) << 8) | uint32_t(m[4 * t + 3]);
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t t1 = hh + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) +
                          kK[t] + w[t];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      hh = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d;
    h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }
}

// The same with the x86 SHA extensions, following the published method of
// Intel's "Intel SHA Extensions" paper (Gulley et al., 2013): the state lives
// as (A,B,E,F) and (C,D,G,H), the register packing sha256rnds2 requires; each
// sha256rnds2 does two rounds, sha256msg1/msg2 extend the message schedule
// four words at a time.
__attribute__((target("sha,sse4.1,ssse3"))) void compress_shani(uint32_t h[8],
                                                                const uint8_t* m,
                                                                size_t nblocks) {
  const __m128i bswap = _mm_set_epi64x(0x0c0d0e0f08090a0bULL, 0x0405060700010203ULL);
  __m128i tmp = _mm_shuffle_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(h)), 0xB1);
  __m128i st1 = _mm_shuffle_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(h + 4)), 0x1B);
  __m128i st0 = _mm_alignr_epi8(tmp, st1, 8);   // A B E F
  st1 = _mm_blend_epi16(st1, tmp, 0xF0);        // C D G H
  for (; nblocks; --nblocks, m += 64) {
    const __m128i save0 = st0, save1 = st1;
    __m128i w[16];
    for (int i = 0; i < 4; ++i)
      w[i] = _mm_shuffle_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i*>(m + 16 * i)),
                              bswap);
    for (int i = 4; i < 16; ++i) {
      __m128i x = _mm_sha256msg1_epu32(w[i - 4], w[i - 3]);
      x = _mm_add_epi32(x, _mm_alignr_epi8(w[i - 1], w[i - 2], 4));
      w[i] = _mm_sha256msg2_epu32(x, w[i - 1]);
    }
    for (int i = 0; i < 16; ++i) {
      __m128i k = _mm_add_epi32(w[i], _mm_loadu_si128(reinterpret_cast<const __m128i*>(kK + 4 * i)));
      st1 = _mm_sha256rnds2_epu32(st1, st0, k);
      k = _mm_shuffle_epi32(k, 0x0E);
      st0 = _mm_sha256rnds2_epu32(st0, st1, k);
    }
    st0 = _mm_add_epi32(st0, save0);
    st1 = _mm_add_epi32(st1, save1);
  }
  tmp = _mm_shuffle_epi32(st0, 0x1B);
  st1 = _mm_shuffle_epi32(st1, 0xB1);
  st0 = _mm_blend_epi16(tmp, st1, 0xF0);
  st1 = _mm_alignr_epi8(st1, tmp, 8);
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h), st0);
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h + 4), st1);
}

// The SHA extensions when the CPU has them, unless PA_SHA256_PORTABLE=1.
bool have_shani() {
  static const bool yes = [] {
    const char* force = std::getenv("PA_SHA256_PORTABLE");
    if (force && force[0] == '1') return false;
    return __builtin_cpu_supports("sha") && __builtin_cpu_supports("sse4.1") &&
           __builtin_cpu_supports("ssse3");
  }();
  return yes;
}

void compress(uint32_t h[8], const uint8_t* m, size_t nblocks) {
  if (have_shani()) {
    compress_shani(h, m, nblocks);
  } else {
    compress_portable(h, m, nblocks);
  }
}

class Sha256 {
 public:
  Sha256() {
    const uint32_t h0[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                            0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
    std::memcpy(h_, h0, sizeof(h_));
  }
  void update(const void* data, size_t len) {
    const uint8_t* d = static_cast<const uint8_t*>(data);
    total_ += len;
    if (fill_) {
      const size_t take = std::min(len, 64 - fill_);
      std::memcpy(buf_ + fill_, d, take);
      fill_ += take;
      d += take;
      len -= take;
      if (fill_ < 64) return;
      compress(h_, buf_, 1);
      fill_ = 0;
    }
    if (len >= 64) {
      compress(h_, d, len / 64);
      d += len / 64 * 64;
      len %= 64;
    }
    std::memcpy(buf_, d, len);
    fill_ = len;
  }
  Hash finish() {
    const uint64_t bits = total_ * 8;
    uint8_t pad[72] = {0x80};
    const size_t padlen = (fill_ < 56 ? 56 : 120) - fill_;
    for (int i = 0; i < 8; ++i) pad[padlen + i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
    update(pad, padlen + 8);
    Hash out;
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = static_cast<uint8_t>(h_[i] >> (24 - 8 * j));
    return out;
  }

 private:
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  uint64_t total_ = 0;
};

inline void le32_at(uint8_t* p, uint32_t v) {
  p[0] = uint8_t(v);
  p[1] = uint8_t(v >> 8);
  p[2] = uint8_t(v >> 16);
  p[3] = uint8_t(v >> 24);
}

// Key of one full block: SHA-256(parent ‖ LE32(n) ‖ tokens as LE32 ‖
// LE32(|extra|) ‖ extra), the message assembled in one buffer.
Hash block_hash(const Hash& parent, const int32_t* tokens, int n, const void* extra,
                size_t extra_len) {
  uint8_t small[512];
  std::vector<uint8_t> big;
  const size_t len = 32 + 4 + 4 * static_cast<size_t>(n) + 4 + extra_len;
  uint8_t* msg = small;
  if (len > sizeof(small)) {
    big.resize(len);
    msg = big.data();
  }
  std::memcpy(msg, parent.data(), 32);
  le32_at(msg + 32, static_cast<uint32_t>(n));
  for (int i = 0; i < n; ++i) le32_at(msg + 36 + 4 * i, static_cast<uint32_t>(tokens[i]));
  le32_at(msg + 36 + 4 * n, static_cast<uint32_t>(extra_len));
  if (extra_len) std::memcpy(msg + 40 + 4 * n, extra, extra_len);
  Sha256 s;
  s.update(msg, len);
  return s.finish();
}

// Request key: LE32(|salt|) ‖ salt ‖ extra.  The first block of a chain
// hashes all of it; later blocks hash only `extra` (the bytes after the salt).
std::string make_key(const void* salt, int salt_len, const void* extra, int extra_len) {
  std::string k(4, '\0');
  const uint32_t n = static_cast<uint32_t>(salt_len);
  for (int i = 0; i < 4; ++i) k[i] = static_cast<char>(n >> (8 * i));
  if (salt_len) k.append(static_cast<const char*>(salt), salt_len);
  if (extra_len) k.append(static_cast<const char*>(extra), extra_len);
  return k;
}

size_t salt_len_of(const std::string& key) {
  uint32_t n = 0;
  for (int i = 0; i < 4; ++i) n |= uint32_t(uint8_t(key[i])) << (8 * i);
  return n;
}

// bytes hashed with block `depth` of a request with this key
void extra_of(const std::string& key, int64_t depth, const void** p, size_t* n) {
  const size_t off = depth == 0 ? 0 : 4 + salt_len_of(key);
  *p = key.data() + off;
  *n = key.size() - off;
}

struct HashOf {
  size_t operator()(const Hash& h) const {
    uint64_t x;
    std::memcpy(&x, h.data(), 8);
    return static_cast<size_t>(x);
  }
};

// ---------------------------------------------------------------------------
// Chain-hash index
// ---------------------------------------------------------------------------
class HashIndex final : public PrefixIndex {
 public:
  explicit HashIndex(int32_t nb) : key_(nb), depth_(nb, 0), idle_at_(nb, 0) {}
  int kind() const override { return PA_PREFIX_HASH; }

  void lookup(const Pool& p, const std::string& key, const int32_t* tokens, int64_t n,
              std::vector<int32_t>& hits, Pos& pos) const override {
    const int32_t bs = p.block_size;
    const int64_t m = n > 0 ? (n - 1) / bs : 0;
    Hash parent{};
    for (int64_t i = 0; i < m; ++i) {
      const void* e;
      size_t el;
      extra_of(key, i, &e, &el);
      const Hash h = block_hash(parent, tokens + i * bs, bs, e, el);
      auto it = map_.find(h);
      if (it == map_.end()) break;
      hits.push_back(it->second);
      parent = h;
    }
    pos.chain = parent;
  }

  void commit(Pool&, int64_t, Seq& s, const std::vector<int32_t>& h, const Pos& pos,
              int64_t queried) override {
    s.chain = pos.chain;
    hits += static_cast<int64_t>(h.size());
    this->queried += queried;
  }

  void add_full_block(Pool& p, int64_t, Seq& s, int32_t b, int64_t depth,
                      const int32_t* tokens) override {
    const void* e;
    size_t el;
    extra_of(s.key, depth, &e, &el);
    s.chain = block_hash(s.chain, tokens, p.block_size, e, el);
    if (map_.count(s.chain) || p.idx[b]) return;  // content already indexed
    map_.emplace(s.chain, b);
    key_[b] = s.chain;
    depth_[b] = depth;
    p.index_hold(b);
  }

  void on_idle(Pool& p, int32_t b) override {
    idle_at_[b] = p.tick;
    idle_.insert(std::make_tuple(p.tick, -depth_[b], b));
  }
  void on_busy(Pool&, int32_t b) override {
    idle_.erase(std::make_tuple(idle_at_[b], -depth_[b], b));
  }

  int64_t evictable(const Pool& p, const std::vector<int32_t>& keep) const override {
    int64_t n = static_cast<int64_t>(idle_.size());
    for (int32_t b : keep)
      if (p.idx[b] && p.seq_refs(b) == 0) --n;
    return n;
  }

  // oldest idle block first; among blocks idle since the same operation, the
  // deepest (the end of a chain goes before its prefix)
  void evict(Pool& p, int64_t k) override {
    while (k > 0 && !idle_.empty()) {
      const int32_t b = std::get<2>(*idle_.begin());
      idle_.erase(idle_.begin());
      map_.erase(key_[b]);
      p.index_drop(b);
      ++evicted;
      --k;
    }
  }

  int64_t indexed() const override { return static_cast<int64_t>(map_.size()); }

 private:
  std::unordered_map<Hash, int32_t, HashOf> map_;
  std::vector<Hash> key_;
  std::vector<int64_t> depth_, idle_at_;
  std::set<std::tuple<int64_t, int64_t, int32_t>> idle_;
};

// ---------------------------------------------------------------------------
// Radix tree index
// ---------------------------------------------------------------------------
class RadixIndex final : public PrefixIndex {
  struct Node {
    int32_t parent = -1;
    bool root = false;
    bool alive = true;
    int64_t depth = 0;               // blocks above this node's first block
    std::vector<int32_t> blocks;     // physical blocks, one per full block of tokens
    std::vector<int32_t> toks;       // blocks.size() * bs token ids
    std::vector<int32_t> kids;       // child nodes (distinct first blocks)
    int64_t busy = 0;                // blocks of this node some sequence holds
    int64_t pins = 0;                // sequences positioned in this node
    int64_t tick = 0;                // last use
    std::unordered_set<int64_t> here;  // ids of the sequences positioned here
  };

 public:
  explicit RadixIndex(int32_t nb) : node_of_(nb, -1), pos_in_(nb, 0) {}
  int kind() const override { return PA_PREFIX_RADIX; }

  void lookup(const Pool& p, const std::string& key, const int32_t* tokens, int64_t n,
              std::vector<int32_t>& hits, Pos& pos) const override {
    const int32_t bs = p.block_size;
    const int64_t m = n > 0 ? (n - 1) / bs : 0;
    auto r = roots_.find(key);
    pos.node = r == roots_.end() ? -1 : r->second;
    pos.off = 0;
    if (pos.node < 0) return;
    int32_t cur = pos.node;
    int64_t i = 0;
    while (i < m) {
      const int32_t c = find_child(cur, tokens + i * bs, bs);
      if (c < 0) break;
      const Node& nd = nodes_[c];
      int32_t j = 0;
      while (j < static_cast<int32_t>(nd.blocks.size()) && i < m &&
             std::equal(tokens + i * bs, tokens + (i + 1) * bs, nd.toks.begin() + j * bs)) {
        hits.push_back(nd.blocks[j]);
        ++j;
        ++i;
      }
      cur = c;
      pos.node = c;
      pos.off = j;
      if (j < static_cast<int32_t>(nd.blocks.size())) break;
    }
  }

  void commit(Pool& p, int64_t id, Seq& s, const std::vector<int32_t>& h, const Pos& pos,
              int64_t queried) override {
    int32_t node = pos.node;
    if (node < 0) {  // first request with this key: a new root
      node = new_node(-1, 0);
      nodes_[node].root = true;
      roots_.emplace(s.key, node);
    }
    for (int32_t x = node; x >= 0; x = nodes_[x].parent) {  // the matched path was used now
      nodes_[x].tick = p.tick;
      refresh(x);
    }
    place(id, s, node, pos.off);
    hits += static_cast<int64_t>(h.size());
    this->queried += queried;
  }

  void add_full_block(Pool& p, int64_t id, Seq& s, int32_t b, int64_t,
                      const int32_t* tokens) override {
    const int32_t bs = p.block_size;
    int32_t x = s.node;
    int32_t off = s.node_off;
    Node* nd = &nodes_[x];
    if (off < static_cast<int32_t>(nd->blocks.size())) {
      if (std::equal(tokens, tokens + bs, nd->toks.begin() + off * bs)) {
        place(id, s, x, off + 1);  // the tree already holds this block's content
        return;
      }
      split(p, x, off);
      nd = &nodes_[x];
    }
    const int32_t c = find_child(x, tokens, bs);
    if (c >= 0) {
      place(id, s, c, 1);
      return;
    }
    if (p.idx[b]) {  // cannot happen: only a sequence's own new block is added
      p.untrack(id, s);
      return;
    }
    if (!nd->root && nd->kids.empty()) {  // extend the leaf
      nd->blocks.push_back(b);
      nd->toks.insert(nd->toks.end(), tokens, tokens + bs);
      hold(p, b, x, static_cast<int32_t>(nd->blocks.size()) - 1);
      nd->tick = p.tick;
      refresh(x);
      place(id, s, x, static_cast<int32_t>(nd->blocks.size()));
      return;
    }
    const int32_t leaf = new_node(x, nd->depth + static_cast<int64_t>(nd->blocks.size()));
    Node& l = nodes_[leaf];
    l.blocks.push_back(b);
    l.toks.assign(tokens, tokens + bs);
    l.tick = p.tick;
    nodes_[x].kids.push_back(leaf);
    refresh(x);
    hold(p, b, leaf, 0);
    refresh(leaf);
    place(id, s, leaf, 1);
  }

  void on_fork(Pool&, int64_t child, Seq& s) override {
    Node& nd = nodes_[s.node];
    ++nd.pins;
    nd.here.insert(child);
    refresh(s.node);
  }

  void untrack(Pool&, int64_t id, Seq& s) override {
    if (s.node < 0) return;
    Node& nd = nodes_[s.node];
    --nd.pins;
    nd.here.erase(id);
    refresh(s.node);
    s.node = -1;
  }

  void on_idle(Pool& p, int32_t b) override {
    Node& nd = nodes_[node_of_[b]];
    if (--nd.busy == 0) nd.tick = p.tick;
    refresh(node_of_[b]);
  }
  void on_busy(Pool&, int32_t b) override {
    ++nodes_[node_of_[b]].busy;
    refresh(node_of_[b]);
  }

  // whole subtrees with no busy block and no positioned sequence can go
  int64_t evictable(const Pool&, const std::vector<int32_t>& keep) const override {
    std::unordered_set<int32_t> kept;
    for (int32_t b : keep)
      for (int32_t x = node_of_[b]; x >= 0; x = nodes_[x].parent) kept.insert(x);
    int64_t total = 0;
    for (const auto& r : roots_) total += free_blocks(r.second, kept).second;
    return total;
  }

  void evict(Pool& p, int64_t k) override {
    while (k > 0 && !cand_.empty()) {
      const int32_t x = std::get<2>(*cand_.begin());
      cand_.erase(cand_.begin());
      Node& nd = nodes_[x];
      for (int32_t b : nd.blocks) {
        node_of_[b] = -1;
        p.index_drop(b);
        ++evicted;
        --k;
      }
      indexed_ -= static_cast<int64_t>(nd.blocks.size());
      nd.alive = false;
      in_cand_[x] = 0;
      Node& par = nodes_[nd.parent];
      par.kids.erase(std::find(par.kids.begin(), par.kids.end(), x));
      --live_;
      refresh(nd.parent);
    }
  }

  int64_t indexed() const override { return indexed_; }
  int64_t nodes() const override { return live_; }

 private:
  int32_t new_node(int32_t parent, int64_t depth) {
    nodes_.emplace_back();
    cand_key_.emplace_back();
    in_cand_.push_back(0);
    Node& n = nodes_.back();
    n.parent = parent;
    n.depth = depth;
    ++live_;
    return static_cast<int32_t>(nodes_.size()) - 1;
  }

  int32_t find_child(int32_t x, const int32_t* tokens, int32_t bs) const {
    for (int32_t c : nodes_[x].kids)
      if (std::equal(tokens, tokens + bs, nodes_[c].toks.begin())) return c;
    return -1;
  }

  void hold(Pool& p, int32_t b, int32_t x, int32_t at) {
    node_of_[b] = x;
    pos_in_[b] = at;
    p.index_hold(b);
    ++indexed_;
    if (p.seq_refs(b) > 0) ++nodes_[x].busy;
  }

  void place(int64_t id, Seq& s, int32_t x, int32_t off) {
    if (s.node != x) {
      if (s.node >= 0) {
        Node& o = nodes_[s.node];
        --o.pins;
        o.here.erase(id);
        refresh(s.node);
      }
      Node& nd = nodes_[x];
      ++nd.pins;
      nd.here.insert(id);
      s.node = x;
      refresh(x);
    }
    s.node_off = off;
  }

  // Node x keeps its first `off` blocks; a new node takes the rest and x's
  // children.  Sequences positioned past `off` move with their blocks.
  void split(Pool& p, int32_t x, int32_t off) {
    const int32_t bs = p.block_size;
    const int32_t y = new_node(x, nodes_[x].depth + off);
    Node& nx = nodes_[x];
    Node& ny = nodes_[y];
    ny.blocks.assign(nx.blocks.begin() + off, nx.blocks.end());
    ny.toks.assign(nx.toks.begin() + static_cast<int64_t>(off) * bs, nx.toks.end());
    ny.kids = std::move(nx.kids);
    ny.tick = nx.tick;
    nx.blocks.resize(off);
    nx.toks.resize(static_cast<size_t>(off) * bs);
    nx.kids.assign(1, y);
    for (int32_t c : ny.kids) nodes_[c].parent = y;
    nx.busy = ny.busy = 0;
    for (int32_t i = 0; i < static_cast<int32_t>(nx.blocks.size()); ++i)
      nx.busy += p.seq_refs(nx.blocks[i]) > 0;
    for (int32_t i = 0; i < static_cast<int32_t>(ny.blocks.size()); ++i) {
      node_of_[ny.blocks[i]] = y;
      pos_in_[ny.blocks[i]] = i;
      ny.busy += p.seq_refs(ny.blocks[i]) > 0;
    }
    std::vector<int64_t> moving;
    for (int64_t id : nx.here) {
      const Seq& s = p.seqs.at(id);
      if (s.node_off > off) moving.push_back(id);
    }
    for (int64_t id : moving) {
      Seq& s = p.seqs.at(id);
      nx.here.erase(id);
      --nx.pins;
      ny.here.insert(id);
      ++ny.pins;
      s.node = y;
      s.node_off -= off;
    }
    refresh(x);
    refresh(y);
  }

  // (blocks freeable under x including x, whether x's whole subtree can go)
  std::pair<bool, int64_t> free_blocks(int32_t x, const std::unordered_set<int32_t>& kept) const {
    const Node& nd = nodes_[x];
    bool all = nd.busy == 0 && nd.pins == 0 && !kept.count(x);
    int64_t total = 0;
    for (int32_t c : nd.kids) {
      auto r = free_blocks(c, kept);
      total += r.second;
      all = all && r.first;
    }
    if (all && !nd.root) total += static_cast<int64_t>(nd.blocks.size());
    return {all, total};
  }

  // eviction candidates: live non-root leaves that no sequence holds or sits
  // in, least recently used first, deeper first among equals
  void refresh(int32_t x) {
    Node& nd = nodes_[x];
    const bool want = nd.alive && !nd.root && nd.kids.empty() && nd.busy == 0 && nd.pins == 0;
    if (in_cand_[x]) {
      cand_.erase(cand_key_[x]);
      in_cand_[x] = 0;
    }
    if (want) {
      cand_key_[x] = std::make_tuple(nd.tick, -nd.depth, x);
      cand_.insert(cand_key_[x]);
      in_cand_[x] = 1;
    }
  }

  std::vector<Node> nodes_;
  std::vector<std::tuple<int64_t, int64_t, int32_t>> cand_key_;
  std::vector<uint8_t> in_cand_;
  std::set<std::tuple<int64_t, int64_t, int32_t>> cand_;
  std::unordered_map<std::string, int32_t> roots_;
  std::vector<int32_t> node_of_, pos_in_;
  int64_t indexed_ = 0, live_ = 0;
};

}  // namespace

std::unique_ptr<PrefixIndex> make_hash_index(int32_t nb) {
  return std::unique_ptr<PrefixIndex>(new HashIndex(nb));
}
std::unique_ptr<PrefixIndex> make_radix_index(int32_t nb) {
  return std::unique_ptr<PrefixIndex>(new RadixIndex(nb));
}

}  // namespace pa

using namespace pa;

PA_EXPORT pa_status pa_sha256(const void* data, size_t len, uint8_t* out) {
  if (!out || (len && !data)) return PA_ERR_INVALID;
  Sha256 s;
  s.update(data, len);
  const Hash h = s.finish();
  std::memcpy(out, h.data(), 32);
  return PA_OK;
}

PA_EXPORT pa_status pa_prefix_block_hash(const uint8_t* parent, const int32_t* tokens, int n,
                                         const void* extra, int extra_len, uint8_t* out) {
  if (!out || n < 0 || extra_len < 0 || (n && !tokens) || (extra_len && !extra))
    return PA_ERR_INVALID;
  Hash par{};
  if (parent) std::memcpy(par.data(), parent, 32);
  const Hash h = block_hash(par, tokens, n, extra, static_cast<size_t>(extra_len));
  std::memcpy(out, h.data(), 32);
  return PA_OK;
}

PA_EXPORT pa_status pa_pool_enable_prefix_cache(pa_pool* p, int kind) {
  if (!p) return PA_ERR_INVALID;
  if (!p->seqs.empty() || p->index) return PA_ERR_INVALID;
  if (kind == PA_PREFIX_HASH) {
    p->index = make_hash_index(p->num_blocks);
  } else if (kind == PA_PREFIX_RADIX) {
    p->index = make_radix_index(p->num_blocks);
  } else {
    return PA_ERR_UNSUPPORTED;
  }
  return PA_OK;
}

PA_EXPORT pa_status pa_seq_create_cached(pa_pool* p, int64_t seq, const int32_t* tokens, int n,
                                         const void* salt, int salt_len, const void* extra,
                                         int extra_len, int* cached_tokens_out,
                                         int64_t* slots_out) {
  if (!p || n < 0 || salt_len < 0 || extra_len < 0) return PA_ERR_INVALID;
  if ((n > 0 && (!tokens || !slots_out)) || (salt_len && !salt) || (extra_len && !extra))
    return PA_ERR_INVALID;
  if (!p->index) return PA_ERR_INVALID;
  if (p->seqs.count(seq)) return PA_ERR_INVALID;
  const int32_t bs = p->block_size;
  const std::string key = make_key(salt, salt_len, extra, extra_len);
  // 1. pure lookup, then the capacity check: nothing changes on failure
  std::vector<int32_t> hits;
  PrefixIndex::Pos pos;
  p->index->lookup(*p, key, tokens, n, hits, pos);
  const int64_t cached = static_cast<int64_t>(hits.size()) * bs;
  const int64_t need = (n - cached + bs - 1) / bs;
  if (need > p->gpu.count + p->index->evictable(*p, hits)) return PA_ERR_NO_BLOCKS;
  // 2. commit
  ++p->tick;
  Seq& s = p->seqs.emplace(seq, Seq()).first->second;
  s.tracked = true;
  s.key = key;
  for (int32_t b : hits) {
    p->retain(b);
    s.table.push_back(b);
  }
  s.fill = cached;
  p->index->commit(*p, seq, s, hits, pos, n > 0 ? (n - 1) / bs : 0);
  if (!p->ensure(need)) return PA_ERR_NO_BLOCKS;  // unreachable after the check above
  for (int64_t t = cached; t < n; ++t) {
    if (t % bs == 0) s.table.push_back(p->alloc());
    slots_out[t - cached] = static_cast<int64_t>(s.table.back()) * bs + t % bs;
    s.fill = t + 1;
    if (s.tracked && t % bs == bs - 1) {
      p->index->add_full_block(*p, seq, s, s.table.back(), t / bs, tokens + (t / bs) * bs);
    }
  }
  if (s.tracked) s.pending.assign(tokens + (n / bs) * bs, tokens + n);
  p->tokens += n;
  if (cached_tokens_out) *cached_tokens_out = static_cast<int>(cached);
  return PA_OK;
}

PA_EXPORT pa_status pa_prefix_stats(const pa_pool* p, int64_t* out) {
  if (!p || !out) return PA_ERR_INVALID;
  if (!p->index) {
    for (int i = 0; i < 6; ++i) out[i] = 0;
    return PA_OK;
  }
  out[0] = p->index->indexed();
  out[1] = p->index->evictable(*p, {});
  out[2] = p->index->hits;
  out[3] = p->index->queried;
  out[4] = p->index->evicted;
  out[5] = p->index->nodes();
  return PA_OK;
}
