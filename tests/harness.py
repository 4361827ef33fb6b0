"""Drive a synth.Scenario through one side: the oracle side (PoolModel + the
oracle's NumPy write/copy) or the GPU side (C++ pool + libpa.so kernels).

The harness only sequences operations; it holds no method arithmetic.  Writes
are batched: pending token writes are flushed before any block copy and before
any free, so the order of effects on the cache is the scenario's order.
"""
from __future__ import annotations

import numpy as np

import synth

FLUSH_TOKENS = 1 << 18

ABS_TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
REL_TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


class OracleSide:
    def __init__(self, sc: synth.Scenario):
        from oracle import attention as A
        from oracle.pool_model import PoolModel
        wl = sc.wl
        self.A = A
        self.wl = wl
        self.pool = PoolModel(sc.num_blocks, wl.block_size, sc.free_order)
        st = synth.STORAGE[wl.dtype]
        self.kc = np.empty(A.k_cache_shape(sc.num_blocks, wl.h_kv, wl.block_size, wl.head_dim,
                                           wl.dtype), dtype=st)
        self.vc = np.empty(A.v_cache_shape(sc.num_blocks, wl.h_kv, wl.block_size, wl.head_dim,
                                           wl.dtype), dtype=st)
        ib = np.uint32 if wl.dtype == "f32" else np.uint16
        self.kc.view(ib)[...] = synth.poison_bits(wl.dtype)
        self.vc.view(ib)[...] = synth.poison_bits(wl.dtype)

    def create(self, s):
        assert self.pool.create(s) == 0

    def fork(self, p, c):
        assert self.pool.fork(p, c) == 0

    def free(self, s):
        assert self.pool.free_seq(s) == 0

    def append(self, seqs, k):
        st, slots, pairs = self.pool.append_batch(list(seqs), k)
        assert st == 0, st
        return np.asarray(slots, dtype=np.int64), np.asarray(pairs, dtype=np.int32).reshape(-1, 2)

    def copy(self, pairs):
        self.A.copy_blocks(self.kc, self.vc, pairs)

    def write(self, slots, kv, vv):
        self.A.write_kv(self.kc, self.vc, kv, vv, slots)

    def enable_swap(self, n):
        assert self.pool.set_host_blocks(n) == 0
        self.kh = np.empty((n,) + self.kc.shape[1:], dtype=self.kc.dtype)
        self.vh = np.empty((n,) + self.vc.shape[1:], dtype=self.vc.dtype)
        ib = np.uint32 if self.wl.dtype == "f32" else np.uint16
        self.kh.view(ib)[...] = synth.poison_bits(self.wl.dtype)
        self.vh.view(ib)[...] = synth.poison_bits(self.wl.dtype)

    def swap_out(self, seqs):
        st, pairs = self.pool.swap_out(list(seqs))
        assert st == 0, st
        self.A.swap_blocks(self.kc, self.vc, self.kh, self.vh, pairs)
        return np.asarray(pairs, dtype=np.int32).reshape(-1, 2)

    def swap_in(self, seqs):
        st, pairs = self.pool.swap_in(list(seqs))
        assert st == 0, st
        self.A.swap_blocks(self.kh, self.vh, self.kc, self.vc, pairs)
        return np.asarray(pairs, dtype=np.int32).reshape(-1, 2)

    def tables(self, seqs):
        ts = [self.pool.block_table(s) for s in seqs]
        maxb = max(1, max(len(t) for t, _ in ts))
        tab = np.full((len(seqs), maxb), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, (t, n) in enumerate(ts):
            tab[i, :len(t)] = t
            lens[i] = n
        return tab, lens

    def decode(self, q, seqs, rows=None):
        tab, lens = self.tables(seqs)
        return self.A.paged_decode(q, self.kc, self.vc, tab, lens, self.wl.scale, self.wl.dtype,
                                   seqs=rows)


class GpuSide:
    def __init__(self, sc: synth.Scenario, guard_blocks: int = 1, stream=None):
        import torch
        from paged_kv_cache_12_amd.manager import PagedKVCache
        wl = sc.wl
        self.wl = wl
        self.torch = torch
        self.stream = stream
        self.cache = PagedKVCache(sc.num_blocks, wl.block_size, wl.h_kv, wl.head_dim, wl.dtype,
                                  free_order=sc.free_order, guard_blocks=guard_blocks,
                                  fill_bits=synth.poison_bits(wl.dtype))
        self.pool = self.cache.pool

    def create(self, s):
        self.cache.create(s)

    def fork(self, p, c):
        self.cache.fork(p, c)

    def free(self, s):
        self.cache.free(s)

    def append(self, seqs, k):
        st, slots, pairs = self.pool.append_batch(np.asarray(seqs, dtype=np.int64), k)
        assert st == 0, st
        return slots.copy(), pairs.copy()

    def _on(self):
        # the inputs' copies and the kernels on the side's stream, in order
        return self.cache._on(self.stream)

    def copy(self, pairs):
        from paged_kv_cache_12_amd import pa_copy_blocks
        with self._on():
            dp = self.torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).cuda()
            pa_copy_blocks(self.cache.k_cache, self.cache.v_cache, dp)

    def write(self, slots, kv, vv):
        from paged_kv_cache_12_amd import pa_write_kv
        from paged_kv_cache_12_amd.manager import storage_to_torch
        t = self.torch
        with self._on():
            ds = t.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
            kd = storage_to_torch(kv, self.wl.dtype).cuda()
            vd = storage_to_torch(vv, self.wl.dtype).cuda()
            pa_write_kv(kd, vd, self.cache.k_cache, self.cache.v_cache, ds)

    def enable_swap(self, n):
        self.cache.enable_swap(n)
        t = self.torch
        ib = t.int32 if self.wl.dtype == "f32" else t.int16
        bits = synth.poison_bits(self.wl.dtype)
        val = bits if bits < (1 << (8 * ib.itemsize - 1)) else bits - (1 << (8 * ib.itemsize))
        self.cache.k_host.view(ib).fill_(val)
        self.cache.v_host.view(ib).fill_(val)

    def swap_out(self, seqs):
        return self.cache.swap_out(seqs, stream=self.stream)

    def swap_in(self, seqs):
        return self.cache.swap_in(seqs, stream=self.stream)

    def tables(self, seqs):
        return self.cache.tables(seqs)

    def decode(self, q_storage, seqs, partition_size, out=None):
        from paged_kv_cache_12_amd.manager import storage_to_torch
        with self._on():
            q = storage_to_torch(q_storage, self.wl.dtype).cuda()
        out, tab, lens = self.cache.decode(q, seqs, self.wl.scale, partition_size, out=out,
                                           stream=self.stream)
        return out, tab, lens


def execute(sc: synth.Scenario, side, log=None):
    """Run the scenario's ops on `side`.  `log` (list) receives
    ("slots", array) / ("pairs", array) records in order."""
    pend_s, pend_k, pend_v = [], [], []
    count = [0]

    def flush():
        if pend_s:
            side.write(np.concatenate(pend_s), np.concatenate(pend_k), np.concatenate(pend_v))
            pend_s.clear(); pend_k.clear(); pend_v.clear()
            count[0] = 0

    def add(slots, kv, vv):
        pend_s.append(slots); pend_k.append(kv); pend_v.append(vv)
        count[0] += len(slots)
        if count[0] >= FLUSH_TOKENS:
            flush()

    def do_append(seqs, k, kv, vv):
        slots, pairs = side.append(seqs, k)
        if log is not None:
            log.append(("slots", slots.copy()))
            log.append(("pairs", pairs.copy()))
        if len(pairs):
            flush()
            side.copy(pairs)
        add(slots, kv, vv)

    for op in sc.ops:
        kind = op[0]
        if kind == "create":
            side.create(op[1])
        elif kind == "fork":
            side.fork(op[1], op[2])
        elif kind == "free":
            flush()
            side.free(op[1])
        elif kind == "append":
            run = op[1]
            if run.ntok == 0:
                continue
            kv, vv = sc.values(run)
            do_append([run.seq], run.ntok, kv, vv)
        elif kind == "append_rr":
            runs = [r for r in op[1] if r.ntok > 0]
            vals = {r.seq: sc.values(r) for r in runs}
            rounds = max((r.ntok for r in runs), default=0)
            for rr in range(rounds):
                live = [r.seq for r in runs if r.ntok > rr]
                kv = np.stack([vals[s][0][rr] for s in live])
                vv = np.stack([vals[s][1][rr] for s in live])
                do_append(live, 1, kv, vv)
        else:
            raise ValueError(kind)
    flush()


def step_append(sc: synth.Scenario, side, log=None):
    """One decode step's append: one new token per decode sequence."""
    slots, pairs = side.append(sc.decode_seqs, 1)
    if log is not None:
        log.append(("slots", slots.copy()))
        log.append(("pairs", pairs.copy()))
    if len(pairs):
        side.copy(pairs)
    side.write(slots, sc.step_k, sc.step_v)


def check_attention(got, ref, dtype, rows):
    """got: float64 [B][H][d] (GPU result upcast), ref: oracle float64.
    Checks max-abs <= ABS_TOL and, per sequence, max-abs <= REL_TOL * max|ref|.
    Returns (max_abs, worst relative ratio)."""
    worst_abs, worst_rel = 0.0, 0.0
    for s in rows:
        err = np.max(np.abs(got[s] - ref[s]))
        scale = np.max(np.abs(ref[s]))
        worst_abs = max(worst_abs, err)
        if scale > 0:
            worst_rel = max(worst_rel, err / scale)
        assert np.all(np.isfinite(got[s])), f"non-finite output in row {s}"
        assert err <= ABS_TOL[dtype], f"seq {s}: max abs err {err}"
        assert err <= REL_TOL[dtype] * scale + 1e-30 or scale == 0, \
            f"seq {s}: err {err} vs rel gate {REL_TOL[dtype] * scale}"
    return worst_abs, worst_rel
