"""GPU parity under a seeded random mix of the pool's operations: one-call
decode steps (pool append, staging copy, copy-on-write, block write, decode;
fp16 / bf16 steps take the cascade whenever forks share 512 or more tokens), forks, frees, swaps out
to pinned host memory and back, and beam steps on a subset of the sequences,
in random order.  Every decode is compared with the oracle's attention over
the oracle pool's tables, every swap's block pairs with the pool model's, and
the caches bit-exactly with the oracle's after every tenth operation and at
the end.  Each feature has its own tests; this one checks that they compose."""
import random
import sys

import numpy as np
import pytest

import synth
import harness as H

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import paged_kv_cache_12_amd as pa
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,part,seed", [("bf16", 0, 1), ("f16", 64, 2), ("bf16", 512, 3),
                                            ("f32", 32, 4)])
def test_random_operation_mix(dtype, part, seed):
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    from test_gpu_parity import small_scenario, to_f64, assert_caches_equal
    say("mix", dtype, part, seed)
    H_q, H_kv, d, bs = 16, 4, 128, 16
    sc = small_scenario(dtype, H_q, H_kv, d, bs, seed=7000 + seed, lens=[700, 530, 90, 300, 17])
    sc.num_blocks = 1200
    sc.free_order = np.random.default_rng(seed).permutation(sc.num_blocks).astype(np.int32)
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    gs.enable_swap(sc.num_blocks)
    os_.enable_swap(sc.num_blocks)

    max_live, max_ctx = 14, 2048
    maxb = max_ctx // bs
    sbytes = pa.pa_decode_step_staging_size(16, maxb)
    hs = [torch.empty(sbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    ds = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(max(pa.pa_decode_cascade_workspace_size(16, H_q, d, max_ctx, part),
                         pa.pa_decode_workspace_size(16, H_q, d, max_ctx, part), 256),
                     dtype=torch.uint8, device="cuda")
    dev = lambda a: storage_to_torch(a, dtype).cuda()
    rng = random.Random(seed)
    live = list(range(len(sc.decode_seqs)))   # on the GPU
    swapped = []                               # in host blocks
    nxt = 100
    counts = dict(step=0, fork=0, free=0, swap_out=0, swap_in=0, beam=0, pairs=0, cascade=0)
    calls = 0

    def attend(seqs, q, out):
        ref = os_.decode(q, list(seqs))
        H.check_attention(to_f64(out, dtype), ref, dtype, range(len(seqs)))

    for op_i in range(60):
        r = rng.random()
        if r < 0.40 and live:
            seqs = rng.sample(live, rng.randint(1, len(live)))
            B = len(seqs)
            kn = synth.normal_array(seed, (op_i, 1), (B, H_kv, d), dtype)
            vn = synth.normal_array(seed, (op_i, 2), (B, H_kv, d), dtype)
            q = synth.normal_array(seed, (op_i, 3), (B, H_q, d), dtype)
            qd = dev(q)
            out = torch.empty_like(qd)
            pa.pa_decode_step(gs.pool, np.asarray(seqs, dtype=np.int64), dev(kn), dev(vn),
                              gs.cache.k_cache, gs.cache.v_cache, qd, out, sc.wl.scale, part,
                              maxb, hs[calls % 2], ds, ws)
            calls += 1
            torch.cuda.synchronize()
            slots, pairs = os_.append(seqs, 1)
            if len(pairs):
                os_.copy(pairs)
            counts["pairs"] += len(pairs)
            os_.write(slots, kn, vn)
            attend(seqs, q, out)
            counts["step"] += 1
            # the grouping the step planned on (the tables after its append)
            tab, lens = os_.tables(seqs)
            if len(pa.pa_cascade_plan(tab, lens, bs, H_q, H_kv, 512)[1]) > 0:
                counts["cascade"] += 1
        elif r < 0.55 and live and len(live) + len(swapped) < max_live:
            p = rng.choice(live)
            gs.fork(p, nxt)
            os_.fork(p, nxt)
            live.append(nxt)
            nxt += 1
            counts["fork"] += 1
        elif r < 0.65 and len(live) + len(swapped) > 3:
            s = rng.choice(live + swapped)
            gs.free(s)
            os_.free(s)
            (live if s in live else swapped).remove(s)
            counts["free"] += 1
        elif r < 0.75 and len(live) > 2:
            seqs = rng.sample(live, rng.randint(1, 2))
            pg = gs.swap_out(seqs)
            po = os_.swap_out(seqs)
            assert np.array_equal(np.asarray(pg).reshape(-1, 2), po), "swap-out pairs differ"
            for s in seqs:
                live.remove(s)
                swapped.append(s)
            counts["swap_out"] += 1
        elif r < 0.85 and swapped:
            seqs = rng.sample(swapped, rng.randint(1, len(swapped)))
            pg = gs.swap_in(seqs)
            po = os_.swap_in(seqs)
            assert np.array_equal(np.asarray(pg).reshape(-1, 2), po), "swap-in pairs differ"
            for s in seqs:
                swapped.remove(s)
                live.append(s)
            counts["swap_in"] += 1
        elif len(live) >= 2 and len(live) + len(swapped) + 2 <= max_live:
            old = rng.sample(live, 2)
            parents = [rng.choice(old) for _ in range(4)]
            news = list(range(nxt, nxt + 4))
            nxt += 4
            B = len(news)
            kn = synth.normal_array(seed, (op_i, 4), (B, H_kv, d), dtype)
            vn = synth.normal_array(seed, (op_i, 5), (B, H_kv, d), dtype)
            q = synth.normal_array(seed, (op_i, 6), (B, H_q, d), dtype)
            qd = dev(q)
            out = torch.empty_like(qd)
            pa.pa_beam_decode_step(gs.pool, old, parents, news, dev(kn), dev(vn),
                                   gs.cache.k_cache, gs.cache.v_cache, qd, out, sc.wl.scale, part,
                                   maxb, hs[calls % 2], ds, ws)
            calls += 1
            torch.cuda.synchronize()
            st, slots, pairs = os_.pool.beam_step(old, parents, news)
            assert st == 0, st
            if pairs:
                os_.copy(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
            counts["pairs"] += len(pairs)
            os_.write(np.asarray(slots, dtype=np.int64), kn, vn)
            attend(news, q, out)
            for s in old:
                live.remove(s)
            live.extend(news)
            counts["beam"] += 1
        if op_i % 10 == 9:
            torch.cuda.synchronize()
            assert_caches_equal(gs, os_)
    torch.cuda.synchronize()
    assert_caches_equal(gs, os_)
    say("  ops", counts)
    assert counts["step"] > 0 and counts["pairs"] > 0
    assert dtype == "f32" or counts["cascade"] > 0   # fp16 / bf16 steps took the cascade
