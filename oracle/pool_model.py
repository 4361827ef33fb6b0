"""Pure-Python model of the paged KV block pool (test infrastructure only).

What the pages fix:
  * KV blocks of a fixed number of tokens; a sequence's logical blocks map to
    physical blocks anywhere in the pool through a per-request block table that
    also records how many positions are filled (vLLM encyclopedia entry,
    tonho.wtf, section "como funciona"; "KV Cache Administration", section
    "How PagedAttention Works", steps 1 and 2).
  * A new physical block is taken only when the previous one is full, so a
    request wastes at most one block (same section; the briefia.fr explainer,
    section "PagedAttention traite la mémoire").
  * Parallel samples map the prompt blocks with a reference count equal to the
    number of holders; a write into the shared last block copies that block and
    only that block (tonho.wtf, "como funciona"; copy-on-write in all three
    explainers).  Everything is expressed with fork, append and free.

What the pages leave open, fixed here so that tables are reproducible bit for
bit (the C++ pool implements the same policy):
  * free list: FIFO; initial order given by the caller; a block whose refcount
    drops to zero goes to the back;
  * free(seq) releases its blocks in logical order;
  * append(seq, k): a copy happens only on the first token of a call, when the
    sequence's fill is not a multiple of block_size and its last block is held
    by another sequence; the appending sequence copies, the last holder writes
    in place;
  * append is all-or-nothing: if the free list cannot cover the call, nothing
    changes and NO_BLOCKS is returned; a batch append is all-or-nothing over the
    whole batch, processed in the order given.

Swapping (tonho.wtf, "a ideia": the cache can be swapped out to CPU RAM;
"como funciona": eviction takes all of a sequence's blocks or none, and a
preempted sequence comes back by swapping in or by recomputing).  Readings:
  * host blocks are a second pool of ids [0, H) with its own FIFO free list
    (initial order 0..H-1) and reference counts;
  * swap_out(seqs) moves the whole batch or nothing: every distinct GPU block
    the batch's tables name (first appearance: sequence order, then logical
    order) gets one host block, so blocks shared inside the batch stay shared
    on the host; each table entry then names the host block and gives up its
    GPU reference (released in the same order); the pairs (gpu, host) are the
    copies the device must make before a released GPU block is reused;
  * swap_in(seqs) is the mirror image: distinct host blocks get new GPU blocks
    in first-appearance order, refcount = references from the batch, host
    references released in order; pairs (host, gpu);
  * a swapped sequence cannot be appended to, forked or decoded; freeing it
    (the recompute choice) releases its host blocks.

Prefix reuse (oracle/prefix_cache.py): an index may hold one reference on a
full block; "shared" and copy-on-write count sequence references only; when
an allocation finds the free list short the index evicts blocks only it
holds (all-or-nothing checks count them as available).
"""
from __future__ import annotations

from collections import deque

OK, INVALID, UNSUPPORTED, NO_BLOCKS, UNKNOWN_SEQ = 0, 1, 2, 3, 4


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("bad pool size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.fill: dict[int, int] = {}
        self.copies = 0
        self.swapped: set[int] = set()
        self.host_free = deque()
        self.host_ref: list[int] = []
        self.idx = [0] * num_blocks        # 1 if the prefix index holds the block
        self.index = None
        self.tick = 0
        self.track: dict[int, object] = {}  # tracking state of sequences (prefix reuse)

    def seq_refs(self, b: int) -> int:
        return self.ref[b] - self.idx[b]

    def _retain(self, b: int):
        self.ref[b] += 1
        if self.idx[b] and self.seq_refs(b) == 1:
            self.index.on_busy(b)

    def _ensure(self, need: int) -> bool:
        if need <= len(self.free):
            return True
        if self.index is None or len(self.free) + self.index.evictable([]) < need:
            return False
        self.index.evict(need - len(self.free))
        return need <= len(self.free)

    def _untrack(self, sid):
        t = self.track.get(sid)
        if t is not None and t.tracked:
            self.index.untrack(sid, t)
        if t is not None:
            t.tracked = False
            t.pending = []

    def set_host_blocks(self, n: int) -> int:
        if n < 0 or self.swapped:
            return INVALID
        self.host_free = deque(range(n))
        self.host_ref = [0] * n
        return OK

    # -- block primitives ----------------------------------------------------
    def _alloc(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        self.idx[b] = 0
        return b

    def _release(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)
        elif self.idx[b] and self.seq_refs(b) == 0:
            self.index.on_idle(b)

    # -- sequence operations -------------------------------------------------
    def create(self, sid: int) -> int:
        if sid in self.tables:
            return INVALID
        self.tables[sid] = []
        self.fill[sid] = 0
        return OK

    def fork(self, parent: int, child: int) -> int:
        if parent not in self.tables:
            return UNKNOWN_SEQ
        if child in self.tables or parent in self.swapped:
            return INVALID
        self.tables[child] = list(self.tables[parent])
        self.fill[child] = self.fill[parent]
        for b in self.tables[child]:
            self._retain(b)
        if parent in self.track:
            self.track[child] = self.track[parent].copy()
            if self.track[child].tracked:
                self.index.on_fork(child, self.track[child])
        return OK

    def free_seq(self, sid: int) -> int:
        self.tick += 1
        if sid not in self.tables:
            return UNKNOWN_SEQ
        self._free_impl(sid)
        return OK

    def _free_impl(self, sid: int):
        self._untrack(sid)
        self.track.pop(sid, None)
        if sid in self.swapped:
            self.swapped.discard(sid)
            for h in self.tables.pop(sid):
                self._host_release(h)
        else:
            for b in self.tables.pop(sid):
                self._release(b)
        del self.fill[sid]
        return OK

    def _host_release(self, h: int):
        self.host_ref[h] -= 1
        if self.host_ref[h] == 0:
            self.host_free.append(h)

    def _batch_ok(self, sids, want_swapped: bool) -> int:
        for s in sids:
            if s not in self.tables:
                return UNKNOWN_SEQ
        for s in sids:
            if (s in self.swapped) != want_swapped:
                return INVALID
        if len(set(sids)) != len(sids):
            return INVALID
        return OK

    def _distinct(self, sids):
        seen = {}
        for s in sids:
            for b in self.tables[s]:
                if b not in seen:
                    seen[b] = len(seen)
        return list(seen)

    def swap_out(self, sids):
        """Returns (status, pairs [(gpu, host), ...])."""
        self.tick += 1
        st = self._batch_ok(sids, False)
        if st != OK:
            return st, []
        blocks = self._distinct(sids)
        if len(blocks) > len(self.host_free):
            return NO_BLOCKS, []
        to_host = {b: self.host_free.popleft() for b in blocks}
        for s in sids:
            self._untrack(s)
        for s in sids:
            new = []
            for b in self.tables[s]:
                self.host_ref[to_host[b]] += 1
                self._release(b)
                new.append(to_host[b])
            self.tables[s] = new
            self.swapped.add(s)
        return OK, [(b, to_host[b]) for b in blocks]

    def swap_in(self, sids):
        """Returns (status, pairs [(host, gpu), ...])."""
        self.tick += 1
        st = self._batch_ok(sids, True)
        if st != OK:
            return st, []
        hosts = self._distinct(sids)
        if not self._ensure(len(hosts)):
            return NO_BLOCKS, []
        to_gpu = {}
        first = {}
        for h in hosts:
            to_gpu[h] = self._alloc()
            first[h] = True
        for s in sids:
            new = []
            for h in self.tables[s]:
                if first[h]:
                    first[h] = False
                else:
                    self._retain(to_gpu[h])
                self._host_release(h)
                new.append(to_gpu[h])
            self.tables[s] = new
            self.swapped.discard(s)
        return OK, [(h, to_gpu[h]) for h in hosts]

    # -- beam search (tonho.wtf "como funciona": beam candidates share blocks
    # and the pattern changes every step) ----------------------------------------
    def beam_step(self, olds, parents, news, tokens=None):
        """New beams fork their parents (old beams), the old beams are freed,
        then one position is appended to each new beam in order.  Returns
        (status, slots, pairs).  Reading: the fork-and-retire part cannot fail
        once checked; a short free list fails only the append."""
        olds, parents, news = list(olds), list(parents), list(news)
        for o in olds:
            if o not in self.tables:
                return UNKNOWN_SEQ, [], []
        if any(o in self.swapped for o in olds) or len(set(olds)) != len(olds):
            return INVALID, [], []
        if len(set(news)) != len(news):
            return INVALID, [], []
        for par, nw in zip(parents, news):
            if par not in olds or (nw in self.tables and nw not in olds):
                return INVALID, [], []
        self.tick += 1
        kids = []
        for par in parents:
            table = list(self.tables[par])
            for b in table:
                self._retain(b)
            tr = self.track[par].copy() if par in self.track else None
            kids.append((table, self.fill[par], tr))
        for o in olds:
            self._free_impl(o)
        for nw, (table, fill, tr) in zip(news, kids):
            self.tables[nw] = table
            self.fill[nw] = fill
            if tr is not None:
                self.track[nw] = tr
                if tr.tracked:
                    self.index.on_fork(nw, tr)
        return self.append_batch(news, 1 if news else 0,
                                 None if tokens is None else [[t] for t in tokens])

    # -- prefix reuse (oracle/prefix_cache.py) -----------------------------------
    def _release_index_ref(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def enable_prefix_cache(self, kind: int) -> int:
        from . import prefix_cache
        return prefix_cache.enable(self, kind)

    def create_cached(self, sid: int, tokens, salt: bytes = b"", extra: bytes = b""):
        from . import prefix_cache
        return prefix_cache.create_cached(self, sid, tokens, salt, extra)

    def append_tokens(self, sids, tokens):
        return self.append_batch(list(sids), len(tokens[0]) if len(sids) else 0, tokens)

    def prefix_stats(self):
        if self.index is None:
            return {"indexed": 0, "evictable": 0, "hits": 0, "queried": 0, "evicted": 0,
                    "nodes": 0}
        return self.index.stats()

    def host_stats(self):
        return {"host_free": len(self.host_free),
                "host_used": sum(1 for r in self.host_ref if r > 0),
                "swapped": len(self.swapped)}

    def _needed(self, sid: int, k: int, ref) -> int:
        """Blocks that append(sid, k) takes, given refcounts `ref`."""
        n = self.fill[sid]
        if k == 0:
            return 0
        need = sum(1 for pos in range(n, n + k) if pos % self.bs == 0)
        if n % self.bs != 0 and ref[self.tables[sid][-1]] > 1:
            need += 1
        return need

    def _seq_ref_view(self):
        return _SeqRefs(self)

    def _append_one_call(self, sid: int, k: int, slots: list, pairs: list):
        table = self.tables[sid]
        for j in range(k):
            n = self.fill[sid]
            if n % self.bs == 0:
                table.append(self._alloc())
            elif j == 0 and self.seq_refs(table[-1]) > 1:
                old = table[-1]
                new = self._alloc()
                pairs.append((old, new))
                self.copies += 1
                self._release(old)
                table[-1] = new
            slots.append(table[-1] * self.bs + n % self.bs)
            self.fill[sid] = n + 1

    def append(self, sid: int, k: int):
        """Returns (status, slots, pairs)."""
        return self.append_batch([sid], k)

    def append_batch(self, sids, k: int, tokens=None):
        """Append k tokens to each sequence of `sids`, in order.  Returns
        (status, slots [len(sids)*k], pairs [(src, dst), ...]).  tokens
        [len(sids)][k] (token ids) keep a tracked sequence feeding the prefix
        index; without them its tracking ends."""
        if k < 0:
            return INVALID, [], []
        self.tick += 1
        for s in sids:
            if s not in self.tables:
                return UNKNOWN_SEQ, [], []
        if any(s in self.swapped for s in sids) or len(set(sids)) != len(sids):
            return INVALID, [], []
        if k == 0 or not sids:
            return OK, [], []
        # dry run of the refcount changes to count the blocks the batch takes
        ref = {}
        need = 0
        seq_ref = self._seq_ref_view()
        for s in sids:
            view = _RefView(seq_ref, ref)
            c = self._needed(s, k, view)
            need += c
            n = self.fill[s]
            if k and n % self.bs != 0 and view[self.tables[s][-1]] > 1:
                ref[self.tables[s][-1]] = view[self.tables[s][-1]] - 1
        if not self._ensure(need):
            return NO_BLOCKS, [], []
        slots, pairs = [], []
        for i, s in enumerate(sids):
            first = self.fill[s]
            start = len(slots)
            self._append_one_call(s, k, slots, pairs)
            if tokens is None:
                self._untrack(s)
                continue
            t = self.track.get(s)
            if t is None or not t.tracked:
                continue
            for j in range(k):
                if not t.tracked:
                    break
                t.pending.append(int(tokens[i][j]))
                if len(t.pending) == self.bs:
                    self.index.add_full_block(s, t, slots[start + j] // self.bs,
                                              (first + j) // self.bs, t.pending)
                    t.pending = []
        return OK, slots, pairs

    # -- queries -------------------------------------------------------------
    def block_table(self, sid: int):
        return list(self.tables[sid]), self.fill[sid]

    def stats(self):
        used = sum(1 for r in self.ref if r > 0)
        shared = sum(1 for b in range(self.num_blocks) if self.seq_refs(b) > 1)
        tokens = sum(self.fill.values())
        return {"free": len(self.free), "used": used, "shared": shared,
                "tokens": tokens, "copies": self.copies}


class _SeqRefs:
    def __init__(self, pool):
        self.pool = pool

    def __getitem__(self, b):
        return self.pool.seq_refs(b)


class _RefView:
    """Refcounts with a sparse overlay of pending changes (dry runs)."""

    def __init__(self, base, overlay):
        self.base, self.overlay = base, overlay

    def __getitem__(self, b):
        return self.overlay.get(b, self.base[b])
