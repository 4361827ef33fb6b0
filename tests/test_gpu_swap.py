"""GPU parity for swapping (pa_swap_blocks through the C ABI, driven by the
C++ pool) against the oracle: host and device caches bit-exact after every
phase, attention after a round trip within the decode tolerance."""
import dataclasses
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


def storage(t, dtype):
    from paged_kv_cache_12_amd.manager import torch_to_storage
    return torch_to_storage(t, dtype)


def ibits(dtype):
    return np.uint32 if dtype == "f32" else np.uint16


@pytest.mark.parametrize("dtype,bs,d,pairs_on_host", [("bf16", 16, 128, False),
                                                      ("f16", 32, 64, True),
                                                      ("f32", 16, 64, False),
                                                      ("bf16", 32, 128, True)])
def test_swap_blocks_bit_exact(dtype, bs, d, pairs_on_host):
    import torch
    from oracle import attention as A
    from paged_kv_cache_12_amd import pa_swap_blocks
    from paged_kv_cache_12_amd.manager import PagedKVCache, storage_to_torch
    say("swap_blocks", dtype, bs, d, "pairs on host" if pairs_on_host else "pairs on device")
    Hkv, nb, nh = 4, 40, 24
    c = PagedKVCache(nb, bs, Hkv, d, dtype, guard_blocks=1, fill_bits=synth.poison_bits(dtype))
    c.enable_swap(nh)
    kd = synth.normal_array(5, (1,), tuple(c.k_full.shape), dtype)
    vd = synth.normal_array(5, (2,), tuple(c.v_full.shape), dtype)
    c.k_full.copy_(storage_to_torch(kd, dtype).cuda())
    c.v_full.copy_(storage_to_torch(vd, dtype).cuda())
    kh = np.empty(tuple(c.k_host.shape), kd.dtype)
    vh = np.empty(tuple(c.v_host.shape), vd.dtype)
    kh.view(ibits(dtype))[...] = synth.poison_bits(dtype)
    vh.view(ibits(dtype))[...] = synth.poison_bits(dtype)
    c.k_host.copy_(storage_to_torch(kh, dtype))
    c.v_host.copy_(storage_to_torch(vh, dtype))
    g = np.random.default_rng(3)
    out_pairs = np.stack([g.choice(nb, 10, replace=False), g.choice(nh, 10, replace=False)],
                         1).astype(np.int32)
    out_pairs[3] = (nb + 5, 2)          # outside the source cache: skipped
    in_pairs = np.stack([out_pairs[:, 1], g.choice(nb, 10, replace=False)], 1).astype(np.int32)
    in_pairs[7] = (1, -1)               # outside the destination cache: skipped

    def put(p):
        t = torch.from_numpy(p)
        return t.pin_memory() if pairs_on_host else t.cuda()

    pa_swap_blocks(c.k_cache, c.v_cache, c.k_host, c.v_host, put(out_pairs))
    torch.cuda.synchronize()
    kdev, vdev = kd[1:1 + nb], vd[1:1 + nb]
    ok = [p for p in out_pairs.tolist() if 0 <= p[0] < nb and 0 <= p[1] < nh]
    A.swap_blocks(kdev, vdev, kh, vh, ok)
    assert np.array_equal(storage(c.k_host, dtype).view(ibits(dtype)), kh.view(ibits(dtype)))
    assert np.array_equal(storage(c.v_host, dtype).view(ibits(dtype)), vh.view(ibits(dtype)))
    pa_swap_blocks(c.k_host, c.v_host, c.k_cache, c.v_cache, put(in_pairs))
    torch.cuda.synchronize()
    ok = [p for p in in_pairs.tolist() if 0 <= p[0] < nh and 0 <= p[1] < nb]
    A.swap_blocks(kh, vh, kdev, vdev, ok)
    assert np.array_equal(storage(c.k_full, dtype).view(ibits(dtype)), kd.view(ibits(dtype)))
    assert np.array_equal(storage(c.v_full, dtype).view(ibits(dtype)), vd.view(ibits(dtype)))



@pytest.mark.parametrize("dtype,bs,d", [("bf16", 16, 128), ("f32", 32, 64)])
def test_swap_blocks_device_to_device(dtype, bs, d):
    """Both caches in device memory (pools of different sizes, one geometry):
    the chosen blocks arrive bit-exact, nothing else of the destination, its
    guard blocks included, changes."""
    import torch
    from oracle import attention as A
    from paged_kv_cache_12_amd import pa_swap_blocks
    from paged_kv_cache_12_amd.manager import PagedKVCache, storage_to_torch
    say("swap_blocks device to device", dtype, bs, d)
    Hkv, na, nb = 4, 30, 18
    a = PagedKVCache(na, bs, Hkv, d, dtype, guard_blocks=1, fill_bits=synth.poison_bits(dtype))
    b = PagedKVCache(nb, bs, Hkv, d, dtype, guard_blocks=1, fill_bits=synth.poison_bits(dtype))
    ka = synth.normal_array(6, (1,), tuple(a.k_full.shape), dtype)
    va = synth.normal_array(6, (2,), tuple(a.v_full.shape), dtype)
    a.k_full.copy_(storage_to_torch(ka, dtype).cuda())
    a.v_full.copy_(storage_to_torch(va, dtype).cuda())
    kb, vb = storage(b.k_full, dtype), storage(b.v_full, dtype)
    g = np.random.default_rng(4)
    pairs = np.stack([g.choice(na, 12, replace=False), g.choice(nb, 12, replace=False)],
                     1).astype(np.int32)
    pa_swap_blocks(a.k_cache, a.v_cache, b.k_cache, b.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    A.swap_blocks(ka[1:1 + na], va[1:1 + na], kb[1:1 + nb], vb[1:1 + nb], pairs.tolist())
    assert np.array_equal(storage(b.k_full, dtype).view(ibits(dtype)), kb.view(ibits(dtype)))
    assert np.array_equal(storage(b.v_full, dtype).view(ibits(dtype)), vb.view(ibits(dtype)))
    assert np.array_equal(storage(a.k_full, dtype).view(ibits(dtype)), ka.view(ibits(dtype)))


def test_swap_blocks_rejects_pageable_memory():
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import PagedKVCache
    c = PagedKVCache(4, 16, 2, 64, "bf16")
    host_k = torch.empty(tuple(c.k_cache.shape), dtype=torch.bfloat16)   # not pinned
    host_v = torch.empty(tuple(c.v_cache.shape), dtype=torch.bfloat16)
    pairs = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    L = pa.lib()
    st = L.pa_swap_blocks(c.k_cache.data_ptr(), c.v_cache.data_ptr(), 4, host_k.data_ptr(),
                          host_v.data_ptr(), 4, pairs.data_ptr(), 1, 2, 64, 16, pa.PA_BF16,
                          torch.cuda.current_stream().cuda_stream)
    assert st == pa.PA_ERR_INVALID
    torch.cuda.synchronize()


def _host_equal(gs, os_):
    import torch
    torch.cuda.synchronize()
    ib = ibits(gs.wl.dtype)
    assert np.array_equal(storage(gs.cache.k_host, gs.wl.dtype).view(ib), os_.kh.view(ib))
    assert np.array_equal(storage(gs.cache.v_host, gs.wl.dtype).view(ib), os_.vh.view(ib))


@pytest.mark.parametrize("name,batch,ctx_hi", [("opt13b_sampling_cow_fp16", 16, 200),
                                               ("llama3_8b_gqa_bf16", 24, 700),
                                               ("tiny_mha_fp32", None, None)])
def test_swap_round_trip_matches_oracle(name, batch, ctx_hi):
    import torch
    from test_gpu_parity import assert_caches_equal, to_f64
    wl = synth.WORKLOADS[name]
    say("swap round trip", name, batch, ctx_hi)
    # every other sample of a family is swapped out, so the samples that come
    # back hold private copies of their prompt blocks: twice the usual pool
    sc0 = synth.build_scenario(wl, batch=batch, ctx_hi=ctx_hi)
    wl = dataclasses.replace(wl, pool_blocks=2 * sc0.num_blocks)
    sc = synth.build_scenario(wl, batch=batch, ctx_hi=ctx_hi)
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    for side in (gs, os_):
        side.enable_swap(sc.num_blocks)
    seqs = list(sc.decode_seqs)
    out_set, stay = seqs[::2], seqs[1::2]
    # 1. swap out every other sequence (splits sampling families)
    pg, po = gs.swap_out(out_set), os_.swap_out(out_set)
    assert np.array_equal(np.asarray(pg).reshape(-1, 2), po)
    _host_equal(gs, os_)
    assert_caches_equal(gs, os_)
    # 2. the others grow into the released blocks
    k = wl.block_size + 3
    kv = synth.normal_array(wl.seed, (77, 1), (len(stay) * k, wl.h_kv, wl.head_dim), wl.dtype)
    vv = synth.normal_array(wl.seed, (77, 2), (len(stay) * k, wl.h_kv, wl.head_dim), wl.dtype)
    for side in (gs, os_):
        slots, pairs = side.append(stay, k)
        if len(pairs):
            side.copy(pairs)
        side.write(slots, kv, vv)
    assert_caches_equal(gs, os_)
    # 3. swap back in, in another order
    pg, po = gs.swap_in(out_set[::-1]), os_.swap_in(out_set[::-1])
    assert np.array_equal(np.asarray(pg).reshape(-1, 2), po)
    torch.cuda.synchronize()
    assert_caches_equal(gs, os_)
    _host_equal(gs, os_)
    assert gs.pool.host_stats() == os_.pool.host_stats()
    # 4. decode everyone
    out, tab, lens = gs.decode(sc.q, seqs, wl.partition)
    torch.cuda.synchronize()
    tab_o, lens_o = os_.tables(seqs)
    assert np.array_equal(tab[:, :tab_o.shape[1]], tab_o) and np.array_equal(lens, lens_o)
    rows = list(range(len(seqs)))
    ref = os_.decode(sc.q, seqs, rows)
    ea, er = H.check_attention(to_f64(out, wl.dtype), ref, wl.dtype, rows)
    say("  max abs", ea, "max rel", er)


def test_manager_on_a_side_stream_matches_oracle():
    """Every manager operation on a stream that is not the current one: the
    fill, an append with copy-on-write through PagedKVCache.append, swap out
    and back in, and the decode.  Their metadata is copied on that stream, so
    each kernel reads what the pool decided for it."""
    import torch
    from test_gpu_parity import assert_caches_equal, to_f64
    from paged_kv_cache_12_amd.manager import storage_to_torch
    wl = synth.WORKLOADS["opt13b_sampling_cow_fp16"]
    say("manager on a side stream", wl.name)
    sc0 = synth.build_scenario(wl, batch=16, ctx_hi=200)
    wl = dataclasses.replace(wl, pool_blocks=2 * sc0.num_blocks)
    sc = synth.build_scenario(wl, batch=16, ctx_hi=200)
    side = torch.cuda.Stream()
    gs, os_ = H.GpuSide(sc, stream=side), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    for s in (gs, os_):
        s.enable_swap(sc.num_blocks)
    seqs = list(sc.decode_seqs)
    # one token each through the manager's append (forked samples copy first)
    kv = synth.normal_array(wl.seed, (78, 1), (len(seqs), wl.h_kv, wl.head_dim), wl.dtype)
    vv = synth.normal_array(wl.seed, (78, 2), (len(seqs), wl.h_kv, wl.head_dim), wl.dtype)
    with torch.cuda.stream(side):
        kd = storage_to_torch(kv, wl.dtype).cuda()
        vd = storage_to_torch(vv, wl.dtype).cuda()
    slots, pairs = gs.cache.append(seqs, 1, kd, vd, stream=side)
    st, oslots, opairs = os_.pool.append_batch(seqs, 1)
    assert st == 0 and list(slots) == list(oslots)
    assert np.array_equal(np.asarray(pairs).reshape(-1, 2), np.asarray(opairs).reshape(-1, 2))
    if len(opairs):
        os_.copy(opairs)
    os_.write(oslots, kv, vv)
    out_set = seqs[::2]
    pg, po = gs.swap_out(out_set), os_.swap_out(out_set)
    assert np.array_equal(np.asarray(pg).reshape(-1, 2), po)
    pg, po = gs.swap_in(out_set[::-1]), os_.swap_in(out_set[::-1])
    assert np.array_equal(np.asarray(pg).reshape(-1, 2), po)
    out, tab, lens = gs.decode(sc.q, seqs, wl.partition)
    side.synchronize()
    torch.cuda.synchronize()
    assert_caches_equal(gs, os_)
    _host_equal(gs, os_)
    rows = list(range(len(seqs)))
    ref = os_.decode(sc.q, seqs, rows)
    ea, er = H.check_attention(to_f64(out, wl.dtype), ref, wl.dtype, rows)
    say("  max abs", ea, "max rel", er)
