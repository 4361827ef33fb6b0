"""GPU parity for beam search: per-step fork / retire / append with batched
copy-on-write through the C++ pool and the GPU kernels, against the pool model
and the oracle, caches bit-exact after every step, attention every few steps."""
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


@pytest.mark.parametrize("dtype,bs,part,W", [("f16", 16, 512, 4), ("bf16", 32, 0, 3),
                                             ("f32", 16, 64, 2)])
def test_beam_search_matches_oracle(dtype, bs, part, W):
    import torch
    from oracle import attention as A
    from oracle.pool_model import PoolModel
    from paged_kv_cache_12_amd.manager import PagedKVCache, storage_to_torch, torch_to_storage
    from test_gpu_parity import to_f64
    say("beam search", dtype, bs, part, "width", W)
    rng = random.Random(bs * 10 + W)
    Hq, Hkv, d = (4, 4, 64) if dtype == "f32" else (16, 4, 128)
    prompts = 6
    N = 400
    order = np.random.default_rng(W).permutation(N).astype(np.int32)
    gpu = PagedKVCache(N, bs, Hkv, d, dtype, free_order=order, guard_blocks=1,
                       fill_bits=synth.poison_bits(dtype))
    model = PoolModel(N, bs, order)
    st = synth.STORAGE[dtype]
    kc = np.empty(A.k_cache_shape(N, Hkv, bs, d, dtype), st)
    vc = np.empty(A.v_cache_shape(N, Hkv, bs, d, dtype), st)
    ib = np.uint32 if dtype == "f32" else np.uint16
    kc.view(ib)[...] = synth.poison_bits(dtype)
    vc.view(ib)[...] = synth.poison_bits(dtype)

    def dev(a):
        return storage_to_torch(a, dtype).cuda()

    beams, nxt = {}, 0
    for g in range(prompts):
        n = rng.randint(20, 300)
        kv = synth.normal_array(31, (g, 1), (n, Hkv, d), dtype)
        vv = synth.normal_array(31, (g, 2), (n, Hkv, d), dtype)
        gpu.create(nxt)
        gpu.append([nxt], n, dev(kv), dev(vv))
        model.create(nxt)
        s_, slots, _ = model.append(nxt, n)
        A.write_kv(kc, vc, kv, vv, np.asarray(slots))
        beams[g] = [nxt]
        nxt += 1
    copies = 0
    for step in range(12):
        for g in range(prompts):
            old = beams[g]
            parents = [rng.choice(old) for _ in range(W)]
            new = list(range(nxt, nxt + W))
            nxt += W
            kv = synth.normal_array(32, (step, g, 1), (W, Hkv, d), dtype)
            vv = synth.normal_array(32, (step, g, 2), (W, Hkv, d), dtype)
            sl_g, pr_g = gpu.beam_step(old, parents, new, dev(kv), dev(vv))
            so, sl_o, pr_o = model.beam_step(old, parents, new)
            assert so == 0 and sl_g.tolist() == sl_o
            assert [tuple(x) for x in pr_g.tolist()] == pr_o
            if pr_o:
                A.copy_blocks(kc, vc, pr_o)
            A.write_kv(kc, vc, kv, vv, np.asarray(sl_o))
            copies += len(pr_o)
            beams[g] = new
        torch.cuda.synchronize()
        kf, vf = torch_to_storage(gpu.k_full, dtype), torch_to_storage(gpu.v_full, dtype)
        assert np.array_equal(kf[1:1 + N].view(ib), kc.view(ib)), step
        assert np.array_equal(vf[1:1 + N].view(ib), vc.view(ib)), step
        if step % 4 == 3:
            live = [b for g in range(prompts) for b in beams[g]]
            q = synth.normal_array(33, (step,), (len(live), Hq, d), dtype)
            out, tab, lens = gpu.decode(dev(q), live, 1.0 / np.sqrt(d), part)
            torch.cuda.synchronize()
            tab_o = np.full(tab.shape, -1, np.int32)
            lens_o = np.zeros(len(live), np.int32)
            for i, s_ in enumerate(live):
                tb, n = model.block_table(s_)
                tab_o[i, :len(tb)] = tb
                lens_o[i] = n
            assert np.array_equal(tab, tab_o) and np.array_equal(lens, lens_o)
            ref = A.paged_decode(q, kc, vc, tab_o, lens_o, 1.0 / np.sqrt(d), dtype)
            rows = list(range(len(live)))
            ea, er = H.check_attention(to_f64(out, dtype), ref, dtype, rows)
            say("  step", step, "beams", len(live), "copies so far", copies, "max abs", ea)
    assert copies > 0


@pytest.mark.parametrize("dtype,part,kind", [("bf16", 0, 0), ("f16", 64, 0), ("bf16", 64, 1),
                                             ("f16", 0, 2)])
def test_beam_decode_step_matches_oracle(dtype, part, kind):
    """One-call beam steps against the pool model and the oracle.  kind > 0:
    the prompts come through a prefix index (1 chain hash, 2 radix tree)
    and each step passes the new positions' token ids, so the index keeps
    tracking the beams; its statistics equal the model's at the end."""
    import torch
    import paged_kv_cache_12_amd as pa
    from oracle import attention as A
    from oracle.pool_model import PoolModel
    from paged_kv_cache_12_amd.manager import PagedKVCache, storage_to_torch, torch_to_storage
    from test_gpu_parity import to_f64
    say("beam_decode_step", dtype, part, kind)
    rng = random.Random(77 + part)
    Hq, Hkv, d, bs, W, P = 16, 4, 128, 16, 3, 4
    N = 256
    order = np.random.default_rng(5).permutation(N).astype(np.int32)
    gpu = PagedKVCache(N, bs, Hkv, d, dtype, free_order=order, guard_blocks=1,
                       fill_bits=synth.poison_bits(dtype))
    model = PoolModel(N, bs, order)
    st = synth.STORAGE[dtype]
    kc = np.empty(A.k_cache_shape(N, Hkv, bs, d, dtype), st)
    vc = np.empty(A.v_cache_shape(N, Hkv, bs, d, dtype), st)
    ib = np.uint16
    kc.view(ib)[...] = synth.poison_bits(dtype)
    vc.view(ib)[...] = synth.poison_bits(dtype)

    def dev(a):
        return storage_to_torch(a, dtype).cuda()

    beams = []
    if kind:
        gpu.enable_prefix_cache(kind)
        assert model.enable_prefix_cache(kind) == 0
        system = [rng.randrange(1000) for _ in range(40)]
    for g in range(P):
        n = rng.randint(5, 200)
        if kind:
            t = system[:rng.randint(16, 40)] + [rng.randrange(1000) for _ in range(n)]
            kvs = {}

            def k_of(a, b, t=t, kvs=kvs):
                kvs["k"], kvs["v"] = synth.prefix_values(t, a, b, Hkv, d, dtype)
                return dev(kvs["k"])

            c = gpu.create_cached(g, t, k_of, lambda a, b, kvs=kvs: dev(kvs["v"]))
            so, co, slots = model.create_cached(g, t)
            assert so == 0 and co == c
            if len(slots):
                A.write_kv(kc, vc, kvs["k"], kvs["v"], np.asarray(slots))
        else:
            kv = synth.normal_array(41, (g, 1), (n, Hkv, d), dtype)
            vv = synth.normal_array(41, (g, 2), (n, Hkv, d), dtype)
            gpu.create(g)
            gpu.append([g], n, dev(kv), dev(vv))
            model.create(g)
            _, slots, _ = model.append(g, n)
            A.write_kv(kc, vc, kv, vv, np.asarray(slots))
        beams.append(g)
    maxb = 32
    sbytes = pa.pa_decode_step_staging_size(P * W, maxb)
    hs = [torch.empty(sbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    ds = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    nxt = P
    copies = 0
    for step in range(10):
        parents = [rng.choice(beams) for _ in range(P * W)] if step else \
            [b for b in beams for _ in range(W)]
        news = list(range(nxt, nxt + len(parents)))
        nxt += len(parents)
        B = len(news)
        kn = synth.normal_array(42, (step, 1), (B, Hkv, d), dtype)
        vn = synth.normal_array(42, (step, 2), (B, Hkv, d), dtype)
        q = synth.normal_array(42, (step, 3), (B, Hq, d), dtype)
        qd = dev(q)
        out = torch.empty_like(qd)
        toks = [rng.randrange(1000) for _ in news] if kind else None
        pa.pa_beam_decode_step(gpu.pool, beams, parents, news, dev(kn), dev(vn), gpu.k_cache,
                               gpu.v_cache, qd, out, 1.0 / np.sqrt(d), part, maxb,
                               hs[step % 2], ds, ws, tokens=toks)
        torch.cuda.synchronize()
        so, sl_o, pr_o = model.beam_step(beams, parents, news, toks)
        assert so == 0
        if pr_o:
            A.copy_blocks(kc, vc, pr_o)
        copies += len(pr_o)
        A.write_kv(kc, vc, kn, vn, np.asarray(sl_o))
        tab = np.full((B, maxb), -1, np.int32)
        lens = np.zeros(B, np.int32)
        for i, s_ in enumerate(news):
            tb, n = model.block_table(s_)
            tab[i, :len(tb)] = tb
            lens[i] = n
        ref = A.paged_decode(q, kc, vc, tab, lens, 1.0 / np.sqrt(d), dtype)
        H.check_attention(to_f64(out, dtype), ref, dtype, range(B))
        beams = news
    kf, vf = torch_to_storage(gpu.k_full, dtype), torch_to_storage(gpu.v_full, dtype)
    assert np.array_equal(kf[1:1 + N].view(ib), kc.view(ib))
    assert np.array_equal(vf[1:1 + N].view(ib), vc.view(ib))
    assert copies > 0
    if kind:
        ps = model.prefix_stats()
        assert gpu.pool.prefix_stats() == ps and ps["hits"] > 0 and ps["indexed"] > 0
