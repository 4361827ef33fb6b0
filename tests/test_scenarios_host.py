"""The workload scripts run through the C++ host pool (with the oracle's data
operations) and through the pool model give identical slots, pairs, tables and
caches.  CPU only; shrunk sizes."""
import numpy as np
import pytest

import synth
import harness as H
import paged_kv_cache_12_amd as pa


class HostPoolSide(H.OracleSide):
    """The oracle's data operations driven by the C++ pool."""

    def __init__(self, sc):
        super().__init__(sc)
        self.cpool = pa.Pool(sc.num_blocks, sc.wl.block_size, sc.free_order)

    def create(self, s):
        assert self.cpool.create(s) == 0

    def fork(self, p, c):
        assert self.cpool.fork(p, c) == 0

    def free(self, s):
        assert self.cpool.free(s) == 0

    def append(self, seqs, k):
        st, slots, pairs = self.cpool.append_batch(seqs, k)
        assert st == 0
        return slots.copy(), pairs.copy()


SHRINK = {
    "tiny_mha_fp32": dict(),
    "llama3_8b_gqa_bf16": dict(batch=6, ctx_hi=900),
    "opt13b_sampling_fp16": dict(batch=8, ctx_hi=40),
    "opt13b_sampling_cow_fp16": dict(batch=8, ctx_hi=40),
    "long_70b_gqa_bf16": dict(batch=2, ctx_hi=33000),
    "shared_prefix_bf16": dict(batch=6, ctx_hi=100),
}


@pytest.mark.parametrize("name", list(SHRINK))
def test_scenario_host_pool_matches_model(name):
    wl = synth.WORKLOADS[name]
    sc = synth.build_scenario(wl, **SHRINK[name])
    a, b = H.OracleSide(sc), HostPoolSide(sc)
    la, lb = [], []
    H.execute(sc, a, la)
    H.execute(sc, b, lb)
    if wl.step_append:
        H.step_append(sc, a, la)
        H.step_append(sc, b, lb)
    assert len(la) == len(lb)
    for (ka, xa), (kb, xb) in zip(la, lb):
        assert ka == kb and np.array_equal(np.asarray(xa).reshape(-1), np.asarray(xb).reshape(-1))
    assert np.array_equal(a.kc.view(np.uint8), b.kc.view(np.uint8))
    assert np.array_equal(a.vc.view(np.uint8), b.vc.view(np.uint8))
    ta, lna = a.tables(sc.decode_seqs)
    tb, lnb = b.cpool.block_tables(sc.decode_seqs, ta.shape[1])
    assert np.array_equal(ta, tb) and np.array_equal(lna, lnb)
    if name == "opt13b_sampling_cow_fp16":
        assert sum(len(x) for k, x in la if k == "pairs") == 3 * (len(sc.decode_seqs) // 4)
    if name == "opt13b_sampling_fp16":
        assert sum(len(x) for k, x in la if k == "pairs") == 0
    # a decode row through the oracle is finite (unfilled slots are never read)
    out = a.decode(sc.q, sc.decode_seqs, rows=[len(sc.decode_seqs) - 1])
    assert np.all(np.isfinite(out[-1]))
