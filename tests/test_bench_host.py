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


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    bench = _bench()
    base = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    p = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "DECODE_SRC", [str(p)])
    p.write_text(base)
    h0 = bench.source_hash()
    p.write_text(base.replace("// one", "// another comment").replace("  return", "\treturn"))
    assert bench.source_hash() == h0
    p.write_text(base.replace("x + 1", "x + 2"))
    assert bench.source_hash() != h0


def test_cpu_baseline_workers_end_normally():
    """The oracle baseline's worker processes exit by themselves (exit code
    0) instead of being terminated by a signal when the pool closes."""
    bench = _bench()
    sc = synth.build_scenario(synth.WORKLOADS["llama3_8b_gqa_bf16"], **SHRINK["llama3_8b_gqa_bf16"])
    res = bench.cpu_baseline(sc, 0.2, 3)
    assert res["kind"] == "oracle" and res["cores"] == 3 and res["value"] > 0
    assert bench.WORKER_EXIT_CODES == [0, 0, 0]


def test_kv_memory_against_hand_worked_numbers():
    """Two sequences of 60 and 17 tokens in blocks of 16 (the pages' 60-token
    example: four blocks, the last one part full), 8 bytes per token: the
    pool holds 6 blocks = 96 slots for 77 tokens; a contiguous allocator
    sized to the longest sequence reserves 2 x 60 = 120 slots."""
    km = _bench().kv_memory(6, 16, 77 * 8.0, 77 * 8.0, [60, 17], 8)
    assert km["paged_slots"] == 96 and km["paged_tokens_distinct"] == 77
    assert km["paged_used_frac"] == round(77 / 96, 4)
    assert km["contiguous_slots"] == 120 and km["contiguous_used_frac"] == round(77 / 120, 4)
    assert km["paged_bytes"] == 768 and km["contiguous_bytes"] == 960
    # a shared prefix is stored once by the pool, once per sequence contiguously
    km = _bench().kv_memory(3, 16, 40 * 8.0, 80 * 8.0, [40, 40], 8)
    assert km["paged_tokens_distinct"] == 40 and km["contiguous_tokens"] == 80


def test_default_line_nests_the_llama_class_record(monkeypatch, capsys):
    """The default run measures the long-context workload and nests the
    Llama-class record (value, step time, roofline, CPU baseline, ...) in
    the same JSON line; --workload alone measures that workload only.  The
    GPU parts are stood in for by records that name their workload."""
    import json
    bench = _bench()
    calls = []

    def fake_run(args, sc, cpu, partition):
        calls.append(sc.wl.name)
        rec = {k: f"{sc.wl.name}:{k}" for k in bench.NESTED_KEYS}
        rec.update(metric="m", config={"workload": sc.wl.name}, cpu_baseline=cpu)
        return rec

    monkeypatch.setattr(bench, "run_workload", fake_run)
    monkeypatch.setattr(bench, "cpu_baseline", lambda sc, s, w: {"sample": sc.wl.name})
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "2", "--warmup", "1"])
    bench.main()
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert calls == ["long_70b_gqa_bf16", "llama3_8b_gqa_bf16"]
    assert line["config"]["workload"] == "long_70b_gqa_bf16"
    nested = line["llama3_8b_gqa_bf16"]
    assert set(nested) == set(bench.NESTED_KEYS)
    assert nested["roofline"] == "llama3_8b_gqa_bf16:roofline"
    assert nested["cpu_baseline"] == {"sample": "llama3_8b_gqa_bf16"}
    calls.clear()
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "shared_prefix_bf16"])
    bench.main()
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert calls == ["shared_prefix_bf16"] and "llama3_8b_gqa_bf16" not in line
