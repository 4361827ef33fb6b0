"""bench.py's host-side pieces.  replay_sample (the setup of the oracle's
timed sample, cpu_baseline) rebuilds a few sequences of a workload, and the
sequences they were forked from, in the oracle's pool and caches: their
lengths and gathered K/V must equal those of the full replay of the
workload's op script (the tests' harness), for plain, forked (parallel
sampling with copy-on-write, shared prefix) and fp32 workloads.  Block ids may
differ (the sample allocates fewer blocks), so the contents are compared."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import synth
import harness as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SHRINK = {
    "tiny_mha_fp32": dict(),
    "llama3_8b_gqa_bf16": dict(batch=6, ctx_hi=900),
    "opt13b_sampling_cow_fp16": dict(batch=8, ctx_hi=40),
    "shared_prefix_bf16": dict(batch=6, ctx_hi=100),
}


def _bench():
    if "bench" in sys.modules:
        return sys.modules["bench"]
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules["bench"] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", list(SHRINK))
def test_replay_sample_matches_full_replay(name):
    from oracle import attention as A
    wl = synth.WORKLOADS[name]
    sc = synth.build_scenario(wl, **SHRINK[name])
    # a sample that skips the first sequence, so that forked children come
    # without their parent in the sample
    samp = sc.decode_seqs[1:5]
    kc, vc, tab, lens = _bench().replay_sample(sc, samp)
    full = H.OracleSide(sc)
    H.execute(sc, full)
    ftab, flens = full.tables(samp)
    assert lens.tolist() == flens.tolist()
    for i in range(len(samp)):
        Ks, Vs = A.gather_sequence(kc, vc, tab[i], int(lens[i]), wl.dtype)
        Kf, Vf = A.gather_sequence(full.kc, full.vc, ftab[i], int(flens[i]), wl.dtype)
        assert np.array_equal(Ks, Kf) and np.array_equal(Vs, Vf), (name, samp[i])
