"""Pins for the prefix-reuse models (oracle/prefix_cache.py): the published
SHA-256 vectors, the pages' worked examples, salting, the chain's dependence on
the whole prefix, equal reuse from the two structures, the eviction rules, and
a content model showing every hit maps exactly the K/V its request would have
computed.  CPU only."""
import hashlib
import json
import os
import random

import pytest

from oracle.pool_model import PoolModel, OK, NO_BLOCKS, INVALID, UNSUPPORTED
from oracle import prefix_cache as PC

GOLD = os.path.join(os.path.dirname(__file__), "golden")
KINDS = [PC.HASH, PC.RADIX]


def test_sha256_published_vectors():
    g = json.load(open(os.path.join(GOLD, "sha256_vectors.json")))
    for v in g["vectors"]:
        msg = v["message"].encode() * v["repeat"]
        assert hashlib.sha256(msg).hexdigest() == v["sha256"]


def pool(kind, n=256, bs=4):
    p = PoolModel(n, bs)
    assert p.enable_prefix_cache(kind) == OK
    return p


@pytest.mark.parametrize("kind", KINDS)
def test_three_users_share_one_copy_of_the_system_prompt(kind):
    # aitalk "RadixAttention"; techtrend "A sensible instance": three users,
    # one system prompt, three different questions -> the prefix is held once
    bs = 4
    p = pool(kind, bs=bs)
    system = list(range(100, 124))                  # 6 full blocks
    questions = [[1, 2, 3, 4, 5], [6, 7, 8], [9, 10, 11, 12, 13, 14, 15]]
    cached = []
    for u, q in enumerate(questions):
        st, c, slots = p.create_cached(u, system + q)
        assert st == OK
        cached.append(c)
        assert len(slots) == len(system) + len(q) - c
    assert cached == [0, 24, 24]
    # the six prefix blocks are the same physical blocks for all three
    assert p.tables[0][:6] == p.tables[1][:6] == p.tables[2][:6]
    assert all(p.seq_refs(b) == 3 for b in p.tables[0][:6])
    # everything else is private
    rest = [set(p.tables[u][6:]) for u in range(3)]
    assert not (rest[0] & rest[1]) and not (rest[0] & rest[2]) and not (rest[1] & rest[2])


@pytest.mark.parametrize("kind", KINDS)
def test_1900_of_2000_tokens_cached_leaves_100_to_compute(kind):
    # aitalk / techtrend, step 1: if 1,900 tokens of a 2,000-token prompt are
    # already present, only the remaining 100 are computed
    p = pool(kind, n=1200, bs=4)
    rng = random.Random(1)
    first = [rng.randrange(32000) for _ in range(1900)]
    assert p.create_cached(0, first)[:2] == (OK, 0)
    second = first + [rng.randrange(32000) for _ in range(100)]
    st, cached, slots = p.create_cached(1, second)
    assert st == OK and cached == 1900 and len(slots) == 100


@pytest.mark.parametrize("kind", KINDS)
def test_salting_keeps_tenants_apart(kind):
    p = pool(kind)
    prompt = list(range(40))
    assert p.create_cached(0, prompt, salt=b"tenant-a")[1] == 0
    assert p.create_cached(1, prompt, salt=b"tenant-b")[1] == 0     # identical prompt, no hit
    assert p.create_cached(2, prompt, salt=b"tenant-a")[1] == 36    # same tenant reuses
    assert p.create_cached(3, prompt)[1] == 0                       # no salt is its own tenant
    assert p.create_cached(4, prompt, salt=b"tenant-a", extra=b"adapter-7")[1] == 0
    assert set(p.tables[0][:9]).isdisjoint(p.tables[1][:9])


def test_chain_key_depends_on_the_whole_prefix():
    a = PC.block_key(None, [1, 2, 3, 4])
    b = PC.block_key(a, [5, 6, 7, 8])
    b2 = PC.block_key(PC.block_key(None, [1, 2, 3, 9]), [5, 6, 7, 8])
    assert b != b2                                  # same block tokens, other parent
    assert PC.block_key(None, [5, 6, 7, 8]) != b    # same tokens at another position
    assert PC.block_key(None, [1, 2, 3, 4], b"x") != a
    assert len({a, b, b2}) == 3 and all(len(k) == 32 for k in (a, b, b2))


@pytest.mark.parametrize("kind", KINDS)
def test_a_block_is_reused_only_after_its_own_prefix(kind):
    p = pool(kind)
    p.create_cached(0, [1, 2, 3, 4, 5, 6, 7, 8, 9])
    # the second block's tokens after a different first block: no hit at all
    assert p.create_cached(1, [9, 9, 9, 9, 5, 6, 7, 8, 1])[1] == 0
    # a prompt that stops inside the cached prefix hits its full blocks only,
    # and never its last token's block
    assert p.create_cached(2, [1, 2, 3, 4, 5, 6])[1] == 4
    assert p.create_cached(3, [1, 2, 3, 4, 5, 6, 7, 8])[1] == 4


def _stream(seed, n_req=60, bs=4):
    rng = random.Random(seed)
    systems = [[rng.randrange(1000) for _ in range(rng.randint(4, 30))] for _ in range(4)]
    reqs = []
    for r in range(n_req):
        base = rng.choice(systems)
        cut = rng.randint(0, len(base))
        toks = base[:cut] + [rng.randrange(1000) for _ in range(rng.randint(0, 12))]
        if reqs and rng.random() < 0.3:           # multi-turn: a previous request grows
            toks = rng.choice(reqs)[1] + [rng.randrange(1000) for _ in range(rng.randint(1, 9))]
        reqs.append((r, toks, rng.choice([b"", b"", b"s1"])))
    return reqs


@pytest.mark.parametrize("seed", range(5))
def test_hash_and_tree_reuse_the_same_prefixes(seed):
    # both pages: the two structures reach the same result
    ph, pr = pool(PC.HASH, n=4096), pool(PC.RADIX, n=4096)
    for sid, toks, salt in _stream(seed):
        a = ph.create_cached(sid, toks, salt)
        b = pr.create_cached(sid, toks, salt)
        assert a == b
    assert ph.tables == pr.tables
    assert ph.prefix_stats()["hits"] == pr.prefix_stats()["hits"] > 0


def test_tree_evicts_least_recently_used_leaves_and_keeps_shared_nodes():
    bs = 4
    p = pool(PC.RADIX, n=40, bs=bs)
    system = list(range(100, 116))                    # 4 blocks, shared
    qs = {u: [u * 10 + i for i in range(9)] for u in (1, 2, 3)}   # 2 full blocks + 1
    for u in (1, 2, 3):
        assert p.create_cached(u, system + qs[u])[0] == OK
    for u in (1, 2, 3):
        p.free_seq(u)                                 # 1 idle first, then 2, then 3
    st = p.prefix_stats()
    assert st["indexed"] == 4 + 3 * 2 and st["evictable"] == 10
    shared_blocks = list(p.tables.get(1, []))
    # a new unrelated request needs more than the free list: leaves go first,
    # least recently used first, and the shared system prompt stays
    free0 = len(p.free)
    assert p.create_cached(9, list(range(900, 900 + 4 * (free0 + 3) + 1)))[0] == OK
    nodes = p.index.nodes
    alive_leaves = [nd for nd in nodes if nd.alive and not nd.root and not nd.kids]
    sys_node = [nd for nd in nodes if nd.alive and nd.toks and nd.toks[0] == system[:bs]]
    assert sys_node, "the shared system-prompt node was evicted before its leaves"
    # user 1's leaf (idle first) went, user 3's (idle last) stayed
    leaf_first = {tuple(nd.toks[0]) for nd in alive_leaves}
    assert tuple(qs[1][:bs]) not in leaf_first and tuple(qs[3][:bs]) in leaf_first
    assert p.prefix_stats()["evicted"] >= 2
    del shared_blocks


def test_hash_evicts_the_end_of_a_chain_before_its_prefix():
    bs = 4
    p = pool(PC.HASH, n=8, bs=bs)
    p.create_cached(0, list(range(17)))               # 4 full blocks indexed + 1 partial
    p.free_seq(0)                                     # all idle at the same tick
    assert p.prefix_stats()["evictable"] == 4
    p.create_cached(1, [500 + i for i in range(4 * 6)])   # needs 6 of 8: 2 evictions
    assert p.prefix_stats()["evicted"] == 2
    # the chain lost its last two blocks and kept the first two
    chain0 = [d for b, d in p.index.depth.items() if b in p.index.key_of and d < 4
              and p.index.key_of[b] in p.index.map and p.index.map[p.index.key_of[b]] == b
              and b not in p.tables[1]]
    assert sorted(chain0) == [0, 1]
    p.free_seq(1)
    assert p.create_cached(2, list(range(9)))[1] == 8      # and still hit


@pytest.mark.parametrize("kind", KINDS)
def test_no_blocks_changes_nothing(kind):
    p = pool(kind, n=10, bs=4)
    p.create_cached(0, list(range(20)))
    p.free_seq(0)
    p.create_cached(1, list(range(100, 112)))
    snap = (list(p.free), list(p.ref), list(p.idx), p.prefix_stats(), p.tick,
            {s: list(t) for s, t in p.tables.items()})
    assert p.create_cached(2, list(range(300, 300 + 4 * 20))) == (NO_BLOCKS, 0, [])
    assert snap == (list(p.free), list(p.ref), list(p.idx), p.prefix_stats(), p.tick,
                    {s: list(t) for s, t in p.tables.items()})


def test_enable_rules():
    p = PoolModel(8, 4)
    assert p.create_cached(0, [1, 2, 3])[0] == INVALID          # no index
    assert p.enable_prefix_cache(7) == UNSUPPORTED
    p.create(5)
    assert p.enable_prefix_cache(PC.HASH) == INVALID            # sequences exist
    q = pool(PC.HASH)
    assert q.enable_prefix_cache(PC.RADIX) == INVALID            # already has one
    assert q.create_cached(0, [1])[0] == OK
    assert q.create_cached(0, [1])[0] == INVALID                 # id exists


class Content:
    """Every slot holds a value determined by the token ids up to and
    including its position (as K/V are, in a real model): a sequence must
    always read back exactly the values of its own token list."""

    def __init__(self, p):
        self.p = p
        self.cells = {}
        self.toks = {}

    @staticmethod
    def value(prefix):
        return hashlib.sha256(repr(prefix).encode()).hexdigest()[:12]

    def create(self, sid, toks, salt):
        st, cached, slots = self.p.create_cached(sid, toks, salt)
        if st != OK:
            return
        self.toks[sid] = list(toks)
        for i, sl in enumerate(slots):
            pos = cached + i
            self.cells[sl] = self.value(toks[:pos + 1])

    def append(self, sids, k, rng):
        tk = [[rng.randrange(1000) for _ in range(k)] for _ in sids]
        st, slots, pairs = self.p.append_tokens(sids, tk)
        if st != OK:
            return
        bs = self.p.bs
        for src, dst in pairs:
            for o in range(bs):
                if src * bs + o in self.cells:
                    self.cells[dst * bs + o] = self.cells[src * bs + o]
        i = 0
        for s, row in zip(sids, tk):
            for t in row:
                self.toks[s].append(t)
                self.cells[slots[i]] = self.value(self.toks[s])
                i += 1

    def fork(self, parent, child):
        if self.p.fork(parent, child) == OK:
            self.toks[child] = list(self.toks[parent])

    def free(self, sid):
        self.p.free_seq(sid)
        del self.toks[sid]

    def check(self):
        bs = self.p.bs
        for s, toks in self.toks.items():
            table, n = self.p.block_table(s)
            assert n == len(toks)
            for pos in range(n):
                assert self.cells[table[pos // bs] * bs + pos % bs] == self.value(toks[:pos + 1])


@pytest.mark.parametrize("kind,seed", [(k, s) for k in KINDS for s in range(3)])
def test_every_hit_holds_what_its_request_would_compute(kind, seed):
    rng = random.Random(seed)
    p = pool(kind, n=160, bs=4)
    c = Content(p)
    stream = _stream(100 + seed, n_req=150)
    live, nxt = [], 1000
    for sid, toks, salt in stream:
        c.create(sid, toks, salt)
        if sid in c.toks:
            live.append(sid)
        r = rng.random()
        if live and r < 0.35:
            s = rng.choice(live); live.remove(s); c.free(s)
        elif live and r < 0.5:
            c.fork(rng.choice(live), nxt)
            if nxt in c.toks:
                live.append(nxt)
            nxt += 1
        elif live and r < 0.8:
            c.append(rng.sample(live, min(len(live), rng.randint(1, 3))), rng.randint(1, 6), rng)
        c.check()
    assert p.prefix_stats()["hits"] > 0 and p.prefix_stats()["evicted"] > 0
