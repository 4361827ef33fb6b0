"""Pins for the pure-Python pool model and the KV-size closed form (CPU only)."""
import json
import math
import os
import random

import pytest

from oracle.pool_model import PoolModel, OK, INVALID, NO_BLOCKS, UNKNOWN_SEQ
from oracle.kv_size import kv_bytes_per_token, kv_bytes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def check_invariants(p: PoolModel):
    # every reference is a table entry and vice versa (host blocks for
    # swapped sequences)
    assert sum(p.ref) == sum(len(t) for s, t in p.tables.items() if s not in p.swapped)
    assert sum(p.host_ref) == sum(len(t) for s, t in p.tables.items() if s in p.swapped)
    assert len(set(p.host_free)) == len(p.host_free)
    assert all(p.host_ref[h] == 0 for h in p.host_free)
    assert sum(1 for r in p.host_ref if r > 0) + len(p.host_free) == len(p.host_ref)
    # free list: distinct, unreferenced; free + used = all blocks
    assert len(set(p.free)) == len(p.free)
    assert all(p.ref[b] == 0 for b in p.free)
    used = sum(1 for r in p.ref if r > 0)
    assert used + len(p.free) == p.num_blocks
    for sid, t in p.tables.items():
        n = p.fill[sid]
        # a block only when the previous one is full: waste < one block
        assert len(t) == -(-n // p.bs)
        assert len(t) * p.bs - n < p.bs or n == 0


def test_golden_trace():
    g = json.load(open(os.path.join(GOLD, "pool_trace.json")))
    p = PoolModel(g["num_blocks"], g["block_size"], g["free_order"])
    for st in g["steps"]:
        op = st["op"]
        if op == "create":
            assert p.create(st["seq"]) == st["status"]
        elif op == "fork":
            assert p.fork(st["parent"], st["child"]) == st["status"]
        elif op == "free":
            assert p.free_seq(st["seq"]) == st["status"]
        elif op == "append":
            status, slots, pairs = p.append(st["seq"], st["k"])
            assert status == st["status"]
            if "slots" in st:
                assert slots == st["slots"]
                assert [list(x) for x in pairs] == st["pairs"]
        elif op == "stats":
            s = p.stats()
            for k in ("free", "used", "shared", "tokens", "copies"):
                assert s[k] == st[k], k
        if "table" in st:
            t, n = p.block_table(st["seq"])
            assert t == st["table"] and n == st["fill"]
        if "free" in st and op != "stats":
            assert list(p.free) == st["free"]
        for b, r in st.get("refs", {}).items():
            assert p.ref[int(b)] == r
        check_invariants(p)


@pytest.mark.parametrize("bs,blocks", [(16, 4), (32, 2)])
def test_sixty_tokens_take_only_the_blocks_they_need(bs, blocks):
    # the explainers' example: a 60-token reply occupies only 60 tokens' worth of blocks
    p = PoolModel(100, bs)
    p.create(0)
    assert p.append(0, 60)[0] == OK
    assert len(p.block_table(0)[0]) == blocks == math.ceil(60 / bs)


def test_new_block_only_when_previous_is_full():
    p = PoolModel(10, 16)
    p.create(0)
    for n in range(1, 49):
        p.append(0, 1)
        assert len(p.block_table(0)[0]) == -(-n // 16)
    assert p.stats()["free"] == 7


def test_parallel_sampling_refcount_and_single_block_copy():
    # prompt blocks mapped in every sample with refcount = number of samples;
    # a write into the shared last block copies that block and only it
    p = PoolModel(64, 16, list(range(64)))
    p.create(0)
    p.append(0, 40)                       # blocks 0, 1, 2 (last one holds 8 tokens)
    for c in (1, 2, 3):
        assert p.fork(0, c) == OK
    assert [p.ref[b] for b in (0, 1, 2)] == [4, 4, 4]
    copies = []
    for s in (0, 1, 2, 3):
        st, slots, pairs = p.append(s, 1)
        copies.append(pairs)
    # three appenders copy (refcount 4 -> 3 -> 2 -> 1), the last writes in place
    assert copies == [[(2, 3)], [(2, 4)], [(2, 5)], []]
    assert [p.ref[b] for b in (0, 1, 2, 3, 4, 5)] == [4, 4, 1, 1, 1, 1]
    assert p.block_table(3)[0] == [0, 1, 2]
    assert p.block_table(0)[0] == [0, 1, 3]
    check_invariants(p)


def test_full_shared_block_is_never_copied():
    p = PoolModel(16, 16)
    p.create(0)
    p.append(0, 32)
    p.fork(0, 1)
    st, slots, pairs = p.append(1, 5)
    assert pairs == [] and p.stats()["copies"] == 0


def test_no_blocks_leaves_pool_unchanged():
    p = PoolModel(4, 16, [3, 1, 0, 2])
    p.create(0)
    p.append(0, 40)
    p.fork(0, 1)
    before = (list(p.free), list(p.ref), {k: list(v) for k, v in p.tables.items()}, dict(p.fill))
    st, slots, pairs = p.append_batch([0, 1], 20)   # needs 2 + 2 blocks (incl. one copy), 1 free
    assert st == NO_BLOCKS and slots == [] and pairs == []
    after = (list(p.free), list(p.ref), {k: list(v) for k, v in p.tables.items()}, dict(p.fill))
    assert before == after


def test_batch_append_counts_copies_in_order():
    # two holders of a partly filled block: only the first appender copies
    p = PoolModel(5, 16, [0, 1, 2, 3, 4])
    p.create(0)
    p.append(0, 20)          # blocks 0, 1
    p.fork(0, 1)
    st, slots, pairs = p.append_batch([0, 1], 1)
    assert st == OK and pairs == [(1, 2)]
    assert slots == [2 * 16 + 4, 1 * 16 + 4]


def test_error_statuses():
    p = PoolModel(4, 16)
    assert p.create(0) == OK
    assert p.create(0) == INVALID
    assert p.fork(5, 6) == UNKNOWN_SEQ
    assert p.fork(0, 0) == INVALID
    assert p.append(9, 1)[0] == UNKNOWN_SEQ
    assert p.append(0, -1)[0] == INVALID
    assert p.append_batch([0, 0], 1)[0] == INVALID
    assert p.free_seq(3) == UNKNOWN_SEQ
    assert p.append(0, 0) == (OK, [], [])


def test_random_ops_keep_invariants():
    rng = random.Random(1234)
    p = PoolModel(200, 16, rng.sample(range(200), 200))
    live = []
    nxt = 0
    for _ in range(5000):
        r = rng.random()
        if r < 0.1 or not live:
            p.create(nxt); live.append(nxt); nxt += 1
        elif r < 0.2:
            par = rng.choice(live)
            p.fork(par, nxt); live.append(nxt); nxt += 1
        elif r < 0.3:
            s = rng.choice(live)
            assert p.free_seq(s) == OK
            live.remove(s)
        else:
            k = rng.randint(1, 40)
            sids = rng.sample(live, min(len(live), rng.randint(1, 4)))
            refs_before = list(p.ref)
            st, slots, pairs = p.append_batch(sids, k)
            if st == OK:
                assert len(slots) == len(sids) * k
                for src, dst in pairs:
                    assert refs_before[src] > 1 and refs_before[dst] == 0
                # slots of one call never collide
                assert len(set(slots)) == len(slots)
            else:
                assert st == NO_BLOCKS
        check_invariants(p)


def test_every_written_slot_is_owned_by_exactly_its_sequence():
    # slots handed out are inside the sequence's own (unshared) last block
    rng = random.Random(99)
    p = PoolModel(300, 16, rng.sample(range(300), 300))
    for s in range(8):
        p.create(s)
        p.append(s, rng.randint(1, 100))
    for c in range(8, 16):
        p.fork(rng.randrange(8), c)
    for _ in range(200):
        s = rng.randrange(16)
        st, slots, pairs = p.append(s, rng.randint(1, 20))
        if st != OK:
            continue
        t, n = p.block_table(s)
        for sl in slots:
            b = sl // 16
            assert b in t
            assert p.ref[b] == 1


# ----------------------------------------------------------------------------
# KV-size closed form against the pages' printed numbers
# ----------------------------------------------------------------------------

def test_kv_size_matches_pages():
    g = json.load(open(os.path.join(GOLD, "kv_size_pages.json")))
    for c in g["cases"]:
        per = kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"])
        assert per == c["exact_bytes"], c["model"]
        for pr in c["printed"]:
            got = kv_bytes(pr["tokens"], c["layers"], c["kv_heads"], c["head_dim"],
                           c["elem_bytes"]) / pr["unit"]
            assert abs(got - pr["value"]) / pr["value"] <= c["tol"], (c["model"], got, pr)


def test_kv_size_factors():
    # each factor enters linearly; the leading 2 is K plus V
    assert kv_bytes_per_token(1, 1, 1, 1) == 2
    assert kv_bytes_per_token(3, 5, 7, 2) == 2 * 3 * 5 * 7 * 2
    # the Llama-3-8B-class page figure: 100,000 tokens are 12.8 million KiB
    assert kv_bytes(100000, 32, 8, 128, 2) == 12_800_000 * 1024


# -- swapping (tonho.wtf "a ideia", "como funciona") ---------------------------

class ContentModel:
    """Token payloads per physical slot, moved by the pairs the pool returns
    exactly as the device would move K/V: a sequence must always read back the
    tokens written for it, in order."""

    def __init__(self, p: PoolModel):
        self.p = p
        self.gpu = {}    # block -> list of bs payloads
        self.host = {}
        self.expect = {}

    def new(self, sid):
        assert self.p.create(sid) == OK
        self.expect[sid] = []

    def fork(self, parent, child):
        if self.p.fork(parent, child) == OK:
            self.expect[child] = list(self.expect[parent])

    def append(self, sids, k, rng):
        st, slots, pairs = self.p.append_batch(sids, k)
        if st != OK:
            return
        for src, dst in pairs:
            self.gpu[dst] = list(self.gpu[src])
        i = 0
        for s in sids:
            for _ in range(k):
                tok = rng.randrange(1 << 30)
                b, o = divmod(slots[i], self.p.bs)
                self.gpu.setdefault(b, [None] * self.p.bs)[o] = tok
                self.expect[s].append(tok)
                i += 1

    def swap_out(self, sids):
        st, pairs = self.p.swap_out(sids)
        for g, h in pairs:
            self.host[h] = list(self.gpu[g])
        return st

    def swap_in(self, sids):
        st, pairs = self.p.swap_in(sids)
        for h, g in pairs:
            self.gpu[g] = list(self.host[h])
        return st

    def free(self, sid):
        assert self.p.free_seq(sid) == OK
        del self.expect[sid]

    def check(self):
        for s, want in self.expect.items():
            table, n = self.p.block_table(s)
            src = self.host if s in self.p.swapped else self.gpu
            got = [src[table[t // self.p.bs]][t % self.p.bs] for t in range(n)]
            assert got == want, s


@pytest.mark.parametrize("seed", range(4))
def test_swap_round_trip_keeps_every_sequence_content(seed):
    rng = random.Random(seed)
    p = PoolModel(96, 8, rng.sample(range(96), 96))
    p.set_host_blocks(64)
    c = ContentModel(p)
    live, nxt = [], 0
    for it in range(1500):
        r = rng.random()
        if r < 0.08 or not live:
            c.new(nxt); live.append(nxt); nxt += 1
        elif r < 0.15:
            c.fork(rng.choice(live), nxt)
            if nxt in p.tables:
                live.append(nxt)
            nxt += 1
        elif r < 0.2:
            s = rng.choice(live); live.remove(s); c.free(s)
        elif r < 0.3:
            c.swap_out(rng.sample(live, min(len(live), rng.randint(1, 4))))
        elif r < 0.4:
            off = [s for s in live if s in p.swapped]
            if off:
                c.swap_in(rng.sample(off, min(len(off), rng.randint(1, 4))))
        else:
            on = [s for s in live if s not in p.swapped]
            if on:
                c.append(rng.sample(on, min(len(on), rng.randint(1, 4))),
                         rng.choice([1, 1, 3, 8, 17]), rng)
        check_invariants(p)
        c.check()


def test_swap_keeps_sharing_inside_a_batch_and_frees_gpu_blocks():
    p = PoolModel(12, 4)
    p.set_host_blocks(12)
    p.create(0)
    p.append(0, 10)                      # 3 blocks, last one half full
    for child in (1, 2, 3):
        p.fork(0, child)                 # refcount 4 on all three
    free_before = len(p.free)
    st, pairs = p.swap_out([0, 1, 2, 3])
    assert st == OK and len(pairs) == 3  # one host block per distinct GPU block
    assert len(p.free) == free_before + 3
    assert all(p.host_ref[h] == 4 for _, h in pairs)
    st, back = p.swap_in([3, 2, 1, 0])
    assert st == OK and len(back) == 3
    assert all(p.ref[g] == 4 for _, g in back)
    assert p.host_stats() == {"host_free": 12, "host_used": 0, "swapped": 0}
    # the shared half-full block still copies on the first divergent append
    st, slots, cow = p.append(1, 1)
    assert st == OK and len(cow) == 1


def test_swapping_part_of_a_family_unshares_only_the_swapped_one():
    p = PoolModel(12, 4)
    p.set_host_blocks(12)
    p.create(0)
    p.append(0, 8)
    p.fork(0, 1)
    st, pairs = p.swap_out([1])
    assert st == OK and len(pairs) == 2
    assert [p.ref[b] for b in p.tables[0]] == [1, 1]   # 0 keeps its blocks
    st, back = p.swap_in([1])
    assert st == OK
    assert set(p.tables[1]).isdisjoint(p.tables[0])    # private copies now
    assert p.stats()["shared"] == 0


def test_swap_no_blocks_leaves_everything_unchanged():
    p = PoolModel(6, 4, [4, 0, 5, 1, 3, 2])
    p.set_host_blocks(2)
    p.create(0)
    p.append(0, 12)
    snap = (list(p.free), list(p.ref), list(p.host_free), list(p.host_ref),
            {s: list(t) for s, t in p.tables.items()}, set(p.swapped))
    assert p.swap_out([0]) == (NO_BLOCKS, [])
    assert snap == (list(p.free), list(p.ref), list(p.host_free), list(p.host_ref),
                    {s: list(t) for s, t in p.tables.items()}, set(p.swapped))
    assert p.swap_in([0]) == (INVALID, [])
    assert p.swap_out([0, 9]) == (UNKNOWN_SEQ, [])


# -- beam search (tonho.wtf "como funciona") ------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_beam_steps_keep_every_beam_content_and_share_ancestry(seed):
    rng = random.Random(seed)
    W, bs = 4, 4
    p = PoolModel(200, bs, rng.sample(range(200), 200))
    c = ContentModel(p)
    c.new(0)
    c.append([0], 10, rng)                   # prompt, last block partly filled
    beams = [0]
    nxt = 1
    for step in range(30):
        parents = [rng.choice(beams) for _ in range(W)]
        news = list(range(nxt, nxt + W))
        nxt += W
        toks = [rng.randrange(1 << 30) for _ in news]
        st, slots, pairs = p.beam_step(beams, parents, news)
        assert st == OK
        # content: children inherit the parent's tokens, copies carry them
        for src, dst in pairs:
            c.gpu[dst] = list(c.gpu[src])
        for nw, par in zip(news, parents):
            c.expect[nw] = list(c.expect[par])
        for b in beams:
            del c.expect[b]
        for nw, sl, tok in zip(news, slots, toks):
            bb, o = divmod(sl, bs)
            c.gpu.setdefault(bb, [None] * bs)[o] = tok
            c.expect[nw].append(tok)
        beams = news
        check_invariants(p)
        c.check()
        # one copy per extra holder of a shared, partly filled last block
        n = p.fill[beams[0]] - 1
        holders = {}
        for par in parents:
            holders[par] = holders.get(par, 0) + 1
        expect_copies = sum(h - 1 for h in holders.values()) if n % bs else 0
        assert len(pairs) == expect_copies
        # beams with a common ancestor share the blocks before the divergence
        assert p.tables[beams[0]][0] == p.tables[beams[-1]][0]
        assert p.ref[p.tables[beams[0]][0]] == W


def test_beam_step_checks_before_changing_anything():
    p = PoolModel(16, 4)
    p.create(0)
    p.append(0, 5)
    p.create(7)
    snap = (list(p.free), list(p.ref), {s: list(t) for s, t in p.tables.items()})
    assert p.beam_step([0, 9], [0], [1])[0] == UNKNOWN_SEQ
    assert p.beam_step([0, 0], [0], [1])[0] == INVALID
    assert p.beam_step([0], [7], [1])[0] == INVALID        # parent not an old beam
    assert p.beam_step([0], [0, 0], [1, 1])[0] == INVALID  # repeated new id
    assert p.beam_step([0], [0], [7])[0] == INVALID        # id of a live non-beam
    assert snap == (list(p.free), list(p.ref), {s: list(t) for s, t in p.tables.items()})
    st, slots, pairs = p.beam_step([0], [0, 0, 0], [0, 1, 2])   # reuse the old id
    assert st == OK and len(slots) == 3 and len(pairs) == 2
    assert p.beam_step([0, 1, 2], [], [])[0] == OK              # all beams retire
    assert set(p.tables) == {7}
