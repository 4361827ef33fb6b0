"""GPU parity in the launch configurations bench.py times, at the workloads'
full sizes: the Llama-3-8B-class and long-context 70B-class decode steps
(pa_decode_step: pool append, one metadata copy, decode with the block write
folded in; split-K partitions and their reduce for the long contexts) and the cascade
decode (pa_decode_cascade with the planner's groups, shared-block flag and
issue order) of the two workloads whose sequences share blocks.  Every row
against the oracle; caches bit-exact."""
import sys

import numpy as np
import pytest

import synth
import harness as H
from test_gpu_parity import _rows, assert_caches_equal, check_rows_streamed, to_f64

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


def _filled(name):
    """The workload drawn and filled on both sides (K/V draws computed once)."""
    wl = synth.WORKLOADS[name]
    sc = synth.build_scenario(wl)
    memo = {}
    orig = sc.values

    def values(run):
        if run.key not in memo:
            memo[run.key] = orig(run)
        return memo[run.key]
    sc.values = values
    gs, os_ = H.GpuSide(sc), H.OracleSide(sc)
    H.execute(sc, gs)
    say("  gpu side filled")
    H.execute(sc, os_)
    say("  oracle side filled")
    memo.clear()
    return wl, sc, gs, os_


@pytest.mark.parametrize("name", ["llama3_8b_gqa_bf16", "long_70b_gqa_bf16"])
def test_decode_step_full_size(name):
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    say("decode step at full size:", name)
    wl, sc, gs, os_ = _filled(name)
    seqs = np.asarray(sc.decode_seqs, dtype=np.int64)
    B = seqs.size
    _, lens0 = gs.cache.tables(list(seqs))
    max_after = int(lens0.max()) + 1
    maxb = -(-max_after // wl.block_size)
    sbytes = pa.pa_decode_step_staging_size(B, maxb)
    h_stage = torch.empty(sbytes, dtype=torch.uint8, pin_memory=True)
    d_stage = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    ws_bytes = max(256, pa.pa_decode_workspace_size(B, wl.h_q, wl.head_dim, max_after,
                                                    wl.partition))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    q = storage_to_torch(sc.q, wl.dtype).cuda()
    k_new = storage_to_torch(sc.step_k, wl.dtype).cuda()
    v_new = storage_to_torch(sc.step_v, wl.dtype).cuda()
    out = torch.empty_like(q)
    pa.pa_decode_step(gs.pool, seqs, k_new, v_new, gs.cache.k_cache, gs.cache.v_cache, q, out,
                      wl.scale, wl.partition, maxb, h_stage, d_stage, ws)
    torch.cuda.synchronize()
    H.step_append(sc, os_)
    assert_caches_equal(gs, os_)
    say("  caches bit-exact after the step")
    rows = _rows(wl, sc)
    ea, er = check_rows_streamed(os_, sc, out, wl.dtype, rows,
                                 chunk=1 if wl.partition else 64)
    say("  rows", len(rows), "max abs", ea, "max rel", er)


@pytest.mark.parametrize("name", ["shared_prefix_bf16", "opt13b_sampling_cow_fp16"])
def test_cascade_decode_full_size(name):
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import storage_to_torch
    say("cascade decode at full size:", name)
    wl, sc, gs, os_ = _filled(name)
    seqs = sc.decode_seqs
    tab, lens = gs.cache.tables(seqs)
    pre, groups, members, mp, mm, mr = pa.pa_cascade_plan(tab, lens, wl.block_size, wl.h_q,
                                                          wl.h_kv, 512)
    assert len(groups) > 0 and mp >= 512
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    max_ctx = int(lens.max())
    ws = torch.zeros(max(256, pa.pa_decode_cascade_workspace_size(len(seqs), wl.h_q, wl.head_dim,
                                                                  max_ctx, wl.partition)),
                     dtype=torch.uint8, device="cuda")
    q = storage_to_torch(sc.q, wl.dtype).cuda()
    out = torch.empty_like(q)
    pa.pa_decode_cascade(out, q, gs.cache.k_cache, gs.cache.v_cache, dev(tab), dev(lens),
                         max_ctx, wl.scale, wl.partition, dev(pre), dev(groups.reshape(-1)),
                         dev(members), mp, mm, mr, ws, flags=pa.PA_DECODE_SHARED_KV,
                         seq_order=dev(pa.pa_decode_order(tab, lens)))
    torch.cuda.synchronize()
    rows = _rows(wl, sc)
    ea, er = check_rows_streamed(os_, sc, out, wl.dtype, rows, chunk=64)
    say("  groups", len(groups), "prefix", mp, "rows", len(rows), "max abs", ea, "max rel", er)
