"""GPU parity for the shared-prefix (cascade) decode: pa_decode_cascade on
workloads whose sequences share physical prefix blocks, against the oracle,
and the automatic use inside pa_decode_step."""
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


def _workload(name):
    if name == "prefix_g4":
        return synth.WORKLOADS["shared_prefix_bf16"], dict(batch=18, ctx_hi=300)
    if name == "prefix_g4_long":    # suffixes up to 2500 tokens: several suffix chunks
        return synth.WORKLOADS["shared_prefix_bf16"], dict(batch=18, ctx_hi=2500)
    if name == "prefix_g4_wide":    # 40 sharers: column groups of 32 and 8 members
        return synth.WORKLOADS["shared_prefix_bf16"], dict(batch=40, ctx_hi=120)
    if name == "cow_g1":
        return synth.WORKLOADS["opt13b_sampling_cow_fp16"], dict(batch=16, ctx_hi=150)
    if name == "prefix_g8_bs32":
        wl = dataclasses.replace(synth.WORKLOADS["shared_prefix_bf16"], name="prefix_g8",
                                 h_q=64, h_kv=8, block_size=32, prefix_len=1000, seed=611)
        return wl, dict(batch=7, ctx_hi=200)
    if name == "prefix_g4_f16_d64":
        wl = dataclasses.replace(synth.WORKLOADS["shared_prefix_bf16"], name="prefix_d64",
                                 dtype="f16", head_dim=64, h_q=16, h_kv=4, prefix_len=777,
                                 seed=612)
        return wl, dict(batch=9, ctx_hi=100)
    if name == "prefix_g4_f16_d64_bs32":   # head dim 64 with block size 32, two tiles
        wl = dataclasses.replace(synth.WORKLOADS["shared_prefix_bf16"], name="prefix_d64_bs32",
                                 dtype="f16", head_dim=64, block_size=32, h_q=16, h_kv=4,
                                 prefix_len=700, seed=615)
        return wl, dict(batch=10, ctx_hi=120)
    if name == "prefix_g16":        # one member per 16-column tile, groups of 2, 2, 1
        wl = dataclasses.replace(synth.WORKLOADS["shared_prefix_bf16"], name="prefix_g16",
                                 h_q=64, h_kv=4, prefix_len=600, seed=613)
        return wl, dict(batch=5, ctx_hi=150)
    if name == "prefix_g2_f16":     # 16 members per group (two tiles), then 5
        wl = dataclasses.replace(synth.WORKLOADS["shared_prefix_bf16"], name="prefix_g2",
                                 dtype="f16", h_q=16, h_kv=8, prefix_len=900, seed=614)
        return wl, dict(batch=21, ctx_hi=130)
    raise ValueError(name)


@pytest.mark.parametrize("name,part", [("prefix_g4", 512), ("prefix_g4", 0), ("prefix_g4", 64),
                                       ("prefix_g4_wide", 512), ("prefix_g4_wide", 32),
                                       ("cow_g1", 512), ("cow_g1", 0), ("prefix_g8_bs32", 96),
                                       ("prefix_g4_f16_d64", 256), ("prefix_g4_f16_d64", 0),
                                       # two-tile prefix passes of 4 and 2 waves; rows whose
                                       # rest spans several chunks go through the reduce
                                       ("prefix_g4", 2048), ("prefix_g4_long", 1024),
                                       ("prefix_g4_long", 512),
                                       # GQA widths 16 and 2 (member = column / G)
                                       ("prefix_g16", 256), ("prefix_g16", 0),
                                       ("prefix_g2_f16", 512), ("prefix_g2_f16", 128),
                                       ("prefix_g4_f16_d64_bs32", 512),
                                       ("prefix_g4_f16_d64_bs32", 64)])
def test_cascade_decode_matches_oracle(name, part):
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    from test_gpu_parity import to_f64
    wl, kw = _workload(name)
    say("cascade", name, part)
    sc = synth.build_scenario(wl, **kw)
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    seqs = sc.decode_seqs
    tab, lens = gs.cache.tables(seqs)
    pre, groups, members, mp, mm, mr = pa.pa_cascade_plan(tab, lens, wl.block_size, wl.h_q,
                                                          wl.h_kv, 64)
    assert len(groups) > 0 and mp > 0
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = storage_to_torch(sc.q, wl.dtype).cuda()
    max_ctx = int(lens.max())
    ws = torch.zeros(max(256, pa.pa_decode_cascade_workspace_size(len(seqs), wl.h_q, wl.head_dim,
                                                                  max_ctx, part)),
                     dtype=torch.uint8, device="cuda")
    order = dev(pa.pa_decode_order(tab, lens))
    out = torch.empty_like(q)
    pa.pa_decode_cascade(out, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens), max_ctx,
                         wl.scale, part, dev(pre), dev(groups.reshape(-1)), dev(members), mp, mm, mr,
                         ws, flags=pa.PA_DECODE_SHARED_KV, seq_order=order)
    plain = torch.empty_like(q)
    ws2 = torch.zeros(max(256, pa.pa_decode_workspace_size(len(seqs), wl.h_q, wl.head_dim,
                                                           max_ctx, part)),
                      dtype=torch.uint8, device="cuda")
    pa.pa_decode(plain, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens), max_ctx,
                 wl.scale, part, workspace=ws2, flags=pa.PA_DECODE_SHARED_KV)
    torch.cuda.synchronize()
    rows = list(range(len(seqs)))
    ref = os_.decode(sc.q, seqs, rows)
    ea, er = H.check_attention(to_f64(out, wl.dtype), ref, wl.dtype, rows)
    eb, _ = H.check_attention(to_f64(plain, wl.dtype), ref, wl.dtype, rows)
    say("  groups", len(groups), "prefix", mp, "cascade max abs", ea, "plain", eb)
    # a second call gives the same bits (deterministic order of the merge)
    again = torch.empty_like(q)
    pa.pa_decode_cascade(again, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens),
                         max_ctx, wl.scale, part, dev(pre), dev(groups.reshape(-1)),
                         dev(members), mp, mm, mr, ws, flags=pa.PA_DECODE_SHARED_KV,
                         seq_order=order)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("name,part,cut", [("prefix_g4", 512, 7), ("prefix_g4", 0, 31),
                                           ("prefix_g4", 64, 1), ("prefix_g16", 256, 13),
                                           ("prefix_g2_f16", 128, 5)])
def test_cascade_prefix_length_off_the_32_grid(name, part, cut):
    """A hand-made plan whose prefix lengths are not multiples of 32 (the
    planner rounds down to 32, the cascade entry point takes any shared run):
    the prefix pass ends in a part group and the rest starts inside one."""
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    from test_gpu_parity import to_f64
    wl, kw = _workload(name)
    say("cascade off-grid prefix", name, part, cut)
    sc = synth.build_scenario(wl, **kw)
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    seqs = sc.decode_seqs
    tab, lens = gs.cache.tables(seqs)
    pre, groups, members, mp, mm, mr = pa.pa_cascade_plan(tab, lens, wl.block_size, wl.h_q,
                                                          wl.h_kv, 64)
    assert len(groups) > 0 and mp > cut
    groups = groups.copy()
    groups[:, 2] -= cut
    pre = np.where(pre > 0, pre - cut, 0).astype(np.int32)
    mp = int(groups[:, 2].max())
    mr = int((lens - pre).max())
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = storage_to_torch(sc.q, wl.dtype).cuda()
    max_ctx = int(lens.max())
    ws = torch.zeros(max(256, pa.pa_decode_cascade_workspace_size(len(seqs), wl.h_q, wl.head_dim,
                                                                  max_ctx, part)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    pa.pa_decode_cascade(out, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens), max_ctx,
                         wl.scale, part, dev(pre), dev(groups.reshape(-1)), dev(members), mp, mm, mr,
                         ws, flags=pa.PA_DECODE_SHARED_KV)
    torch.cuda.synchronize()
    rows = list(range(len(seqs)))
    ref = os_.decode(sc.q, seqs, rows)
    ea, _ = H.check_attention(to_f64(out, wl.dtype), ref, wl.dtype, rows)
    say("  groups", len(groups), "prefix", mp, "max abs", ea)


def test_cascade_with_no_groups_is_plain_decode():
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    wl, kw = _workload("prefix_g4")
    sc = synth.build_scenario(wl, **kw)
    gs = H.GpuSide(sc)
    H.execute(sc, gs)
    tab, lens = gs.cache.tables(sc.decode_seqs)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = storage_to_torch(sc.q, wl.dtype).cuda()
    B, mc = len(sc.decode_seqs), int(lens.max())
    ws = torch.zeros(max(pa.pa_decode_cascade_workspace_size(B, wl.h_q, wl.head_dim, mc, 512),
                         pa.pa_decode_workspace_size(B, wl.h_q, wl.head_dim, mc, 512)),
                     dtype=torch.uint8, device="cuda")
    a, b = torch.empty_like(q), torch.empty_like(q)
    empty = torch.zeros(0, dtype=torch.int32, device="cuda")
    pa.pa_decode_cascade(a, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens), mc,
                         wl.scale, 512, dev(np.zeros(B, np.int32)), empty, empty, 0, 0, mc, ws)
    pa.pa_decode(b, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens), mc, wl.scale,
                 512, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,part", [("bf16", 0), ("f16", 256)])
def test_decode_step_uses_the_cascade_for_long_shared_prefixes(dtype, part):
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    from test_gpu_parity import small_scenario, to_f64, assert_caches_equal
    say("decode_step cascade", dtype, part)
    H_q, H_kv, d, bs = 16, 4, 128, 16
    lens = [700, 37, 900, 5]
    sc = small_scenario(dtype, H_q, H_kv, d, bs, seed=9150 + part, lens=lens)
    # seq 0 and 2 get families: three forks each share 700 / 900 tokens
    sc.ops += [("fork", 0, 4), ("fork", 0, 5), ("fork", 2, 6), ("fork", 2, 7), ("fork", 2, 8)]
    sc.decode_seqs = [0, 1, 2, 3, 4, 5, 6, 7, 8]
    sc.num_blocks += 16
    sc.free_order = np.random.default_rng(2).permutation(sc.num_blocks).astype(np.int32)
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    H.execute(sc, os_)
    seqs = np.array(sc.decode_seqs, dtype=np.int64)
    B = len(seqs)
    maxb = 64
    tab, ln = os_.tables(list(seqs))
    pre, groups, members, mp, _, _ = pa.pa_cascade_plan(tab, ln + 1, bs, H_q, H_kv, 512)
    assert len(groups) == 2 and mp == 896          # the step's plan: two families
    sbytes = pa.pa_decode_step_staging_size(B, maxb)
    hs = [torch.empty(sbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    ds = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(max(pa.pa_decode_cascade_workspace_size(B, H_q, d, maxb * bs, part),
                         pa.pa_decode_workspace_size(B, H_q, d, maxb * bs, part), 256),
                     dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(4)
    for step in range(6):
        kn = synth.cast_storage(rng.standard_normal((B, H_kv, d), dtype=np.float32), dtype)
        vn = synth.cast_storage(rng.standard_normal((B, H_kv, d), dtype=np.float32), dtype)
        q = synth.cast_storage(rng.standard_normal((B, H_q, d), dtype=np.float32), dtype)
        qd = storage_to_torch(q, dtype).cuda()
        out = torch.empty_like(qd)
        pa.pa_decode_step(gs.pool, seqs, storage_to_torch(kn, dtype).cuda(),
                          storage_to_torch(vn, dtype).cuda(), gs.cache.k_cache, gs.cache.v_cache,
                          qd, out, sc.wl.scale, part, maxb, hs[step % 2], ds, ws)
        torch.cuda.synchronize()
        slots, pairs = os_.append(list(seqs), 1)
        if len(pairs):
            os_.copy(pairs)
        os_.write(slots, kn, vn)
        ref = os_.decode(q, list(seqs))
        H.check_attention(to_f64(out, dtype), ref, dtype, range(B))
    assert_caches_equal(gs, os_)
