"""Prefix reuse over the pool model (test infrastructure only): chain hashing
and a radix tree, written from the pages, plain and slow.

What the pages fix:
  * chain hashing (aitalk.it, the chain-hashing paragraph of "Due strati, non
    due rivali"; "KV Cache Administration", "How vLLM Implements Prefix
    Caching"): every completed block gets a key computed from its parent
    block's key, its own token ids and optional extra data, so equal prefixes
    give equal chains; lookup computes the keys in order, a hit reuses the
    block, the first miss allocates blocks for the rest; completed blocks go
    back into the cache;
  * cache salting (aitalk.it, third direction of "Oltre le due tecniche";
    "KV Cache Administration", "Cache salting prevents cross-tenant reuse"):
    a tenant-specific element enters the key, so identical prompts of
    different tenants never share;
  * the radix tree (aitalk.it "RadixAttention: un albero che non dimentica";
    "KV Cache Administration", "How RadixAttention Works", steps 1-4): a
    compressed trie in which each distinct prefix is stored once; match the
    longest prefix, reuse it, insert the unmatched rest; under memory pressure
    evict least recently used leaves and keep shared inner nodes;
  * both reach the same reuse; the difference is structural (both pages).

Readings (where the pages are silent):
  * granularity: whole blocks of block_size tokens; only full blocks are
    indexed, as soon as they are full;
  * a lookup considers only full blocks that end before the prompt's last
    token (that token is always computed);
  * key of block i = SHA-256(key of block i-1, 32 zero bytes for i = 0 ‖
    LE32(block_size) ‖ token ids as LE32 ‖ LE32(|e|) ‖ e) with
    e = LE32(|salt|) ‖ salt ‖ extra for block 0 and e = extra after it; the
    tree has one root per (salt, extra);
  * the index holds one reference on each indexed block; a block whose last
    sequence reference goes is idle; eviction happens only when an allocation
    finds the free list short;
  * hash eviction: single idle blocks, the one idle for longest first; among
    blocks idle since the same operation the deepest first, then the lowest
    id;
  * tree eviction: leaves with no held block and no sequence positioned in
    them, least recently used first (use = matched, inserted into, or last
    held block released), deeper first, then the older node; a node with
    children is never evicted;
  * a sequence keeps its position (node, blocks matched in it) while it is
    tracked; a split moves positions past the split point to the new node;
    node ids count up in creation order (a split's second half is new);
  * a tracked sequence whose next full block is already in the tree (same
    tokens) follows the tree and leaves its own block unindexed; the chain
    index likewise keeps the first block registered for a key.
"""
from __future__ import annotations

import hashlib
import struct

from .pool_model import INVALID, NO_BLOCKS, OK, UNSUPPORTED

HASH, RADIX = 1, 2


def le32(v: int) -> bytes:
    return struct.pack("<I", v & 0xFFFFFFFF)


def block_key(parent: bytes | None, tokens, extra: bytes = b"") -> bytes:
    """Chain key of one full block."""
    parent = bytes(32) if parent is None else parent
    body = b"".join(le32(int(t)) for t in tokens)
    return hashlib.sha256(parent + le32(len(tokens)) + body + le32(len(extra)) + extra).digest()


def request_key(salt: bytes, extra: bytes) -> bytes:
    return le32(len(salt)) + salt + extra


def extra_for(key: bytes, depth: int) -> bytes:
    """Bytes hashed with block `depth`: the whole request key for the first
    block, the extra bytes (after the salt) for later ones."""
    if depth == 0:
        return key
    salt_len = struct.unpack("<I", key[:4])[0]
    return key[4 + salt_len:]


class Track:
    """Tracking state of one sequence."""

    def __init__(self, key: bytes):
        self.tracked = True
        self.pending: list[int] = []
        self.chain = bytes(32)
        self.key = key
        self.node = -1
        self.off = 0

    def copy(self):
        t = Track(self.key)
        t.tracked, t.pending, t.chain = self.tracked, list(self.pending), self.chain
        t.node, t.off = self.node, self.off
        return t


class HashIndexModel:
    kind = HASH

    def __init__(self, pool):
        self.p = pool
        self.map: dict[bytes, int] = {}
        self.key_of: dict[int, bytes] = {}
        self.depth: dict[int, int] = {}
        self.idle: dict[int, int] = {}     # block -> tick it became idle
        self.hits = self.queried = self.evicted = 0

    def lookup(self, key: bytes, tokens):
        bs = self.p.bs
        m = (len(tokens) - 1) // bs if len(tokens) else 0
        parent, hits = bytes(32), []
        for i in range(m):
            h = block_key(parent, tokens[i * bs:(i + 1) * bs], extra_for(key, i))
            if h not in self.map:
                break
            hits.append(self.map[h])
            parent = h
        return hits, parent

    def commit(self, sid, t: Track, hits, pos, queried):
        t.chain = pos
        self.hits += len(hits)
        self.queried += queried

    def add_full_block(self, sid, t: Track, b: int, depth: int, tokens):
        t.chain = block_key(t.chain, tokens, extra_for(t.key, depth))
        if t.chain in self.map or self.p.idx[b]:
            return
        self.map[t.chain] = b
        self.key_of[b] = t.chain
        self.depth[b] = depth
        self.p.idx[b] = 1
        self.p.ref[b] += 1

    def on_idle(self, b):
        self.idle[b] = self.p.tick

    def on_busy(self, b):
        del self.idle[b]

    def on_fork(self, sid, t):
        pass

    def untrack(self, sid, t):
        pass

    def evictable(self, keep):
        return len(self.idle) - sum(1 for b in keep if b in self.idle)

    def evict(self, k):
        while k > 0 and self.idle:
            b = min(self.idle, key=lambda x: (self.idle[x], -self.depth[x], x))
            del self.idle[b]
            del self.map[self.key_of.pop(b)]
            self.p.idx[b] = 0
            self.p._release_index_ref(b)
            self.evicted += 1
            k -= 1

    def stats(self):
        return {"indexed": len(self.map), "evictable": self.evictable([]), "hits": self.hits,
                "queried": self.queried, "evicted": self.evicted, "nodes": 0}


class _Node:
    def __init__(self, parent: int, depth: int):
        self.parent = parent
        self.root = False
        self.alive = True
        self.depth = depth
        self.blocks: list[int] = []
        self.toks: list[list[int]] = []    # one token list per block
        self.kids: list[int] = []
        self.busy = 0
        self.pins = 0
        self.tick = 0
        self.here: set[int] = set()


class RadixIndexModel:
    kind = RADIX

    def __init__(self, pool):
        self.p = pool
        self.nodes: list[_Node] = []
        self.roots: dict[bytes, int] = {}
        self.node_of: dict[int, int] = {}
        self.hits = self.queried = self.evicted = 0

    def _new(self, parent, depth):
        self.nodes.append(_Node(parent, depth))
        return len(self.nodes) - 1

    def _child(self, x, tokens):
        for c in self.nodes[x].kids:
            if self.nodes[c].toks[0] == list(tokens):
                return c
        return -1

    def lookup(self, key, tokens):
        bs = self.p.bs
        m = (len(tokens) - 1) // bs if len(tokens) else 0
        node = self.roots.get(key, -1)
        hits = []
        off = 0
        if node < 0:
            return hits, (node, off)
        cur, i = node, 0
        while i < m:
            c = self._child(cur, tokens[i * bs:(i + 1) * bs])
            if c < 0:
                break
            nd = self.nodes[c]
            j = 0
            while j < len(nd.blocks) and i < m and nd.toks[j] == list(tokens[i * bs:(i + 1) * bs]):
                hits.append(nd.blocks[j])
                j += 1
                i += 1
            cur, node, off = c, c, j
            if j < len(nd.blocks):
                break
        return hits, (node, off)

    def commit(self, sid, t: Track, hits, pos, queried):
        node, off = pos
        if node < 0:
            node = self._new(-1, 0)
            self.nodes[node].root = True
            self.roots[t.key] = node
        x = node
        while x >= 0:
            self.nodes[x].tick = self.p.tick
            x = self.nodes[x].parent
        self._place(sid, t, node, off)
        self.hits += len(hits)
        self.queried += queried

    def _place(self, sid, t, x, off):
        if t.node != x:
            if t.node >= 0:
                o = self.nodes[t.node]
                o.pins -= 1
                o.here.discard(sid)
            nd = self.nodes[x]
            nd.pins += 1
            nd.here.add(sid)
            t.node = x
        t.off = off

    def _hold(self, b, x):
        self.node_of[b] = x
        self.p.idx[b] = 1
        self.p.ref[b] += 1
        if self.p.seq_refs(b) > 0:
            self.nodes[x].busy += 1

    def _split(self, x, off):
        y = self._new(x, self.nodes[x].depth + off)
        nx, ny = self.nodes[x], self.nodes[y]
        ny.blocks, nx.blocks = nx.blocks[off:], nx.blocks[:off]
        ny.toks, nx.toks = nx.toks[off:], nx.toks[:off]
        ny.kids, nx.kids = nx.kids, [y]
        ny.tick = nx.tick
        for c in ny.kids:
            self.nodes[c].parent = y
        nx.busy = sum(1 for b in nx.blocks if self.p.seq_refs(b) > 0)
        ny.busy = sum(1 for b in ny.blocks if self.p.seq_refs(b) > 0)
        for b in ny.blocks:
            self.node_of[b] = y
        for sid in sorted(nx.here):
            t = self.p.track[sid]
            if t.off > off:
                nx.here.discard(sid)
                nx.pins -= 1
                ny.here.add(sid)
                ny.pins += 1
                t.node = y
                t.off -= off

    def add_full_block(self, sid, t: Track, b: int, depth: int, tokens):
        tokens = list(tokens)
        x, off = t.node, t.off
        nd = self.nodes[x]
        if off < len(nd.blocks):
            if nd.toks[off] == tokens:
                self._place(sid, t, x, off + 1)
                return
            self._split(x, off)
            nd = self.nodes[x]
        c = self._child(x, tokens)
        if c >= 0:
            self._place(sid, t, c, 1)
            return
        if not nd.root and not nd.kids:
            nd.blocks.append(b)
            nd.toks.append(tokens)
            self._hold(b, x)
            nd.tick = self.p.tick
            self._place(sid, t, x, len(nd.blocks))
            return
        leaf = self._new(x, nd.depth + len(nd.blocks))
        lf = self.nodes[leaf]
        lf.blocks, lf.toks, lf.tick = [b], [tokens], self.p.tick
        self.nodes[x].kids.append(leaf)
        self._hold(b, leaf)
        self._place(sid, t, leaf, 1)

    def on_fork(self, sid, t):
        nd = self.nodes[t.node]
        nd.pins += 1
        nd.here.add(sid)

    def untrack(self, sid, t):
        if t.node < 0:
            return
        nd = self.nodes[t.node]
        nd.pins -= 1
        nd.here.discard(sid)
        t.node = -1

    def on_idle(self, b):
        nd = self.nodes[self.node_of[b]]
        nd.busy -= 1
        if nd.busy == 0:
            nd.tick = self.p.tick

    def on_busy(self, b):
        self.nodes[self.node_of[b]].busy += 1

    def _free_blocks(self, x, kept):
        nd = self.nodes[x]
        whole = nd.busy == 0 and nd.pins == 0 and x not in kept
        total = 0
        for c in nd.kids:
            w, n = self._free_blocks(c, kept)
            total += n
            whole = whole and w
        if whole and not nd.root:
            total += len(nd.blocks)
        return whole, total

    def evictable(self, keep):
        kept = set()
        for b in keep:
            x = self.node_of[b]
            while x >= 0:
                kept.add(x)
                x = self.nodes[x].parent
        return sum(self._free_blocks(r, kept)[1] for r in self.roots.values())

    def _candidates(self):
        return [i for i, nd in enumerate(self.nodes)
                if nd.alive and not nd.root and not nd.kids and nd.busy == 0 and nd.pins == 0]

    def evict(self, k):
        while k > 0:
            cand = self._candidates()
            if not cand:
                break
            x = min(cand, key=lambda i: (self.nodes[i].tick, -self.nodes[i].depth, i))
            nd = self.nodes[x]
            for b in nd.blocks:
                del self.node_of[b]
                self.p.idx[b] = 0
                self.p._release_index_ref(b)
                self.evicted += 1
                k -= 1
            nd.alive = False
            self.nodes[nd.parent].kids.remove(x)

    def stats(self):
        indexed = sum(len(nd.blocks) for nd in self.nodes if nd.alive)
        live = sum(1 for nd in self.nodes if nd.alive)
        return {"indexed": indexed, "evictable": self.evictable([]), "hits": self.hits,
                "queried": self.queried, "evicted": self.evicted, "nodes": live}


def enable(pool, kind: int) -> int:
    if pool.tables or pool.index is not None:
        return INVALID
    if kind == HASH:
        pool.index = HashIndexModel(pool)
    elif kind == RADIX:
        pool.index = RadixIndexModel(pool)
    else:
        return UNSUPPORTED
    return OK


def create_cached(pool, sid: int, tokens, salt: bytes = b"", extra: bytes = b""):
    """Returns (status, cached_tokens, slots for tokens cached..n-1)."""
    tokens = [int(t) for t in tokens]
    if pool.index is None or sid in pool.tables:
        return INVALID, 0, []
    bs, n = pool.bs, len(tokens)
    key = request_key(salt, extra)
    hits, pos = pool.index.lookup(key, tokens)
    cached = len(hits) * bs
    need = -(-(n - cached) // bs)
    if need > len(pool.free) + pool.index.evictable(hits):
        return NO_BLOCKS, 0, []
    pool.tick += 1
    t = Track(key)
    pool.track[sid] = t
    pool.tables[sid] = []
    pool.fill[sid] = cached
    for b in hits:
        pool._retain(b)
        pool.tables[sid].append(b)
    pool.index.commit(sid, t, hits, pos, (n - 1) // bs if n else 0)
    assert pool._ensure(need)
    table, slots = pool.tables[sid], []
    for pos_t in range(cached, n):
        if pos_t % bs == 0:
            table.append(pool._alloc())
        slots.append(table[-1] * bs + pos_t % bs)
        pool.fill[sid] = pos_t + 1
        if t.tracked and pos_t % bs == bs - 1:
            i = pos_t // bs
            pool.index.add_full_block(sid, t, table[-1], i, tokens[i * bs:(i + 1) * bs])
    if t.tracked:
        t.pending = tokens[(n // bs) * bs:]
    return OK, cached, slots
