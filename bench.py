"""PagedAttention decode benchmark on one MI355X.

One step = the whole decode hot path for one batch, one pa_decode_step call:
the host pool appends one token per sequence (slot mapping and copy-on-write
decisions, C++), block tables / lengths / slots go to the device from a
pinned staging buffer (one of four, used in turn) through a copy kernel on
the stream, pa_copy_blocks runs for any copy-on-write pair, and pa_decode
(partition kernel + log-sum-exp reduce) computes the attention output and
stores the new K/V in the same launch (pa_write_kv first for fp32).  Inputs
are resident in HBM before the timed region starts.

Prints one JSON line.  `value` is the effective KV bandwidth of the whole step
(algorithmic KV bytes read by the step's decode / step time);
`roofline` covers pa_decode alone, timed with HIP events on its stream, cache
cold (the calls cycle through copies of the caches, one per layer, so that
more KV than the L2s and the MALL hold is read between two reads of one
copy), mean of the calls.
The oracle baseline runs first, in processes forked before any GPU use.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
# shader-clock cycles of the spin kernel that keeps the device busy while
# short kernels are queued behind it (about 1 ms at 2.4 GHz)
SPIN_CYCLES = 2_400_000
# the headline line: the long-context 70B-class workload (the largest that the
# 70 %-of-peak target names); the Llama-3-8B-class step is measured in the same
# run and nested in the line under its own name
DEFAULT_WORKLOAD = "long_70b_gqa_bf16"
DEFAULT_ALSO = "llama3_8b_gqa_bf16"
# --swap moves half of this workload's sequences out and back
SWAP_WORKLOAD = "llama3_8b_gqa_bf16"
# keys of a nested workload record
NESTED_KEYS = ("value", "unit", "ms_per_step", "pct_of_hbm_peak", "seq_steps_per_s", "dtype",
               "config", "decode_ms_mean", "decode_cold_copies",
               "decode_ms_per_call_p10_median_p90", "host_us_per_step", "copy_blocks",
               "roofline", "read_ceiling", "kv_memory", "cpu_baseline")
# the decode kernels' code: their source and the library headers with device
# code or structures they use (the public header only declares the ABI)
DECODE_SRC = [os.path.join(ROOT, "paged_kv_cache_12_amd", "csrc", f)
              for f in ("pa_decode.hip", "pa_internal.h", "pa_kv_store.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(synth.WORKLOADS),
                    help=f"decode workload (default {DEFAULT_WORKLOAD}; {SWAP_WORKLOAD} for --swap)")
    ap.add_argument("--also", default=None, choices=sorted(synth.WORKLOADS) + ["none"],
                    help="a second workload measured in the same run and nested in the line "
                         f"(default: {DEFAULT_ALSO} with the default --workload, else none)")
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="processes for the oracle baseline (default: host cores, <= 16)")
    ap.add_argument("--swap", action="store_true",
                    help="measure swapping half of the workload's sequences out to pinned "
                         "host memory and back (pa_seq_swap_out/in + pa_swap_blocks)")
    ap.add_argument("--beam", action="store_true",
                    help="measure beam-search steps (fork / retire / append with batched "
                         "copy-on-write, block write, decode) on the OPT-13B-class shapes")
    ap.add_argument("--prefix", action="store_true",
                    help="measure prefix reuse (chain hashing and radix tree) on a shared "
                         "system-prompt request stream (host only)")
    ap.add_argument("--calibrate", action="store_true",
                    help="run only a 1 GiB device copy and fill of known size (for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def calibrate():
    """Known-size traffic for counter calibration: 5 x (fill 1 GiB), then
    5 x (copy 1 GiB -> 1 GiB), then the decode's own load types over 1 GiB:
    pa_read_probe reading every 4 KiB tile once in a random order with
    16-byte loads, 5 x non-temporal then 5 x plain (each launch reads exactly
    1 GiB and writes 128 KiB of per-wave partials)."""
    import torch
    import paged_kv_cache_12_amd as pa
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    del dst
    tile = 4096
    g = torch.Generator().manual_seed(2025)
    order = torch.randperm(n // tile, generator=g).to(torch.int32).cuda()
    partials = torch.empty(16 * pa.pa_read_probe_partials(), dtype=torch.uint8, device="cuda")
    for nt in (True, False):
        for _ in range(5):
            pa.pa_read_probe(src, tile, order, partials, nt)
        torch.cuda.synchronize()
    print(json.dumps({"calibrate": True, "fill_bytes_written": n, "copy_bytes_read": n,
                      "copy_bytes_written": n, "probe_bytes_read": n,
                      "probe_bytes_written": len(partials), "launches_each": 5}), flush=True)


def source_hash() -> str:
    """Hash of the decode kernels' code with comments and whitespace removed:
    the counters in profiles/ stay attached to the code they were taken on,
    and an edit of comments alone does not detach them."""
    h = hashlib.sha256()
    for path in DECODE_SRC:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


class StagingFence:
    """Marks when a step's pinned staging buffer may be refilled: a HIP event
    recorded after the step, created with hipEventDisableSystemFence.  The
    host only needs to know that the step's work has finished (its copy
    kernel has read the buffer), not to see device memory, so the event skips
    the system-scope release (a cache write-back between the decode and the
    next step's copy, about 1.6 us per step here).  The HIP runtime is the
    one already loaded in the process (torch's), so streams are shared."""

    _hip = None

    @classmethod
    def _runtime(cls):
        import ctypes
        if cls._hip is None:
            loaded = re.findall(r"\S*/libamdhip64\.so[.\d]*", open("/proc/self/maps").read())
            cls._hip = ctypes.CDLL(loaded[0] if loaded else "libamdhip64.so.7")
        return cls._hip

    def __init__(self, stream):
        import ctypes
        hip = self._runtime()
        self._h = ctypes.c_void_p()
        flags = 0x2 | 0x20000000  # hipEventDisableTiming | hipEventDisableSystemFence
        if hip.hipEventCreateWithFlags(ctypes.byref(self._h), ctypes.c_uint(flags)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        if hip.hipEventRecord(self._h, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if self._runtime().hipEventSynchronize(self._h) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def __del__(self):
        if self._h and self._hip is not None:
            self._hip.hipEventDestroy(self._h)


def read_ceiling(pa, torch, dev, stream, runs: int = 10):
    """The decode's access pattern without the math: pa_read_probe over 4 GiB
    of random 4 KiB tiles (each read once per run), timed with HIP events on
    the launch stream; GB/s with non-temporal and with plain 16-byte loads."""
    tile, total = 4096, 4 << 30
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    g = torch.Generator().manual_seed(2024)
    order = torch.randperm(total // tile, generator=g).to(torch.int32).to(dev)
    partials = torch.empty(16 * pa.pa_read_probe_partials(), dtype=torch.uint8, device=dev)
    res = {}
    for nt in (True, False):
        for _ in range(2):
            pa.pa_read_probe(buf, tile, order, partials, nt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(runs):
            pa.pa_read_probe(buf, tile, order, partials, nt)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / runs
        res["nontemporal_GBps" if nt else "plain_GBps"] = round(total / (ms * 1e-3) / 1e9, 1)
    del buf, order, partials
    return res


def fill_cache(sc, cache, dev):
    """Run the workload's op script through the product path (C++ pool +
    pa_copy_blocks + pa_write_kv)."""
    import torch
    from paged_kv_cache_12_amd.manager import storage_to_torch
    dt = sc.wl.dtype

    def put(a):
        return storage_to_torch(a, dt).to(dev)

    for op in sc.ops:
        kind = op[0]
        if kind == "create":
            cache.create(op[1])
        elif kind == "fork":
            cache.fork(op[1], op[2])
        elif kind == "free":
            torch.cuda.synchronize()
            cache.free(op[1])
        elif kind == "append":
            run = op[1]
            if run.ntok:
                kv, vv = sc.values(run)
                cache.append([run.seq], run.ntok, put(kv), put(vv))
        elif kind == "append_rr":
            runs = [r for r in op[1] if r.ntok > 0]
            vals = {r.seq: sc.values(r) for r in runs}
            for rr in range(max((r.ntok for r in runs), default=0)):
                live = [r.seq for r in runs if r.ntok > rr]
                kv = np.stack([vals[s][0][rr] for s in live])
                vv = np.stack([vals[s][1][rr] for s in live])
                cache.append(live, 1, put(kv), put(vv))
    torch.cuda.synchronize()


def cascade_plan(pa, torch, dev, tab_h, len_h, wl, part, flags):
    """Shared-prefix plan for a decode over these tables (None when no group
    of sequences shares 512 or more tokens of blocks, or blocks are not
    shared at all)."""
    if not flags or wl.dtype == "f32":
        return None
    pre, groups, members, mp, mm, mr = pa.pa_cascade_plan(tab_h, len_h, wl.block_size, wl.h_q,
                                                          wl.h_kv, 512)
    if len(groups) == 0:
        return None
    put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return {"prefix": put(pre), "groups": put(groups.reshape(-1)), "members": put(members),
            "max_prefix": mp, "max_members": mm, "max_rest": mr, "ngroups": len(groups)}


def run_decode(pa, out, q, cache, d_tab, d_len, max_ctx, wl, part, ws, flags, order, plan):
    kc, vc = cache if isinstance(cache, tuple) else (cache.k_cache, cache.v_cache)
    if plan is None:
        pa.pa_decode(out, q, kc, vc, d_tab, d_len, max_ctx, wl.scale, part, workspace=ws,
                     flags=flags, seq_order=order)
    else:
        pa.pa_decode_cascade(out, q, kc, vc, d_tab, d_len, max_ctx, wl.scale, part,
                             plan["prefix"], plan["groups"], plan["members"], plan["max_prefix"],
                             plan["max_members"], plan["max_rest"], ws, flags=flags,
                             seq_order=order)


def unique_kv_bytes(tables, lens, wl):
    """KV bytes of the distinct physical blocks the batch reads (a block
    aliased by several sequences counts once, with its filled positions)."""
    seen = {}
    bs = wl.block_size
    for row, n in zip(tables, lens):
        nb = -(-int(n) // bs)
        for j in range(nb):
            b = int(row[j])
            fill = min(bs, int(n) - j * bs)
            seen[b] = max(seen.get(b, 0), fill)
    return float(sum(seen.values())) * 2 * wl.h_kv * wl.head_dim * synth.ELEM_BYTES[wl.dtype]


def kv_memory(used_blocks: int, block_size: int, unique_bytes: float, logical_bytes: float,
              lens, token_bytes: int) -> dict:
    """KV memory of the batch as the pool holds it, beside a contiguous
    allocator that reserves the longest context for every sequence (the
    pre-paging systems the pages describe reserve the maximum length per
    request and cannot share a prefix).  Fractions of reserved slots that
    hold a token."""
    slots = int(used_blocks) * block_size
    distinct = unique_bytes / token_bytes
    logical = logical_bytes / token_bytes
    reserved = len(lens) * int(max(lens)) if len(lens) else 0
    return {"paged_slots": slots, "paged_tokens_distinct": round(distinct),
            "paged_used_frac": round(distinct / slots, 4) if slots else None,
            "contiguous_slots": reserved, "contiguous_tokens": round(logical),
            "contiguous_used_frac": round(logical / reserved, 4) if reserved else None,
            "paged_bytes": slots * token_bytes, "contiguous_bytes": reserved * token_bytes}


def host_cores() -> int:
    """Host cores this process may use (the box gives one GPU 16 of them)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_SAMPLE = {}
# exit codes of the last cpu_baseline's worker processes (0: ended normally)
WORKER_EXIT_CODES: list = []


def _oracle_rows(rows):
    """Worker body: the oracle's paged_decode on some rows of the sample."""
    from oracle import attention as A
    t = _SAMPLE
    A.paged_decode(t["q"], t["kc"], t["vc"], t["tab"], t["lens"], t["scale"], t["dtype"],
                   seqs=rows)
    return len(rows)


def replay_sample(sc, samp):
    """The oracle's pool model and caches for the sequences `samp` of a
    workload: its op script replayed for them and the sequences they were
    forked from (creates, forks, frees, appends, copy-on-write copies).
    Returns (k_cache, v_cache, tables [len(samp)][maxb], lengths)."""
    from oracle import attention as A
    from oracle.pool_model import PoolModel
    wl = sc.wl
    model = PoolModel(sc.num_blocks, wl.block_size, sc.free_order)
    st = synth.STORAGE[wl.dtype]
    kc = np.zeros(A.k_cache_shape(sc.num_blocks, wl.h_kv, wl.block_size, wl.head_dim, wl.dtype), st)
    vc = np.zeros(A.v_cache_shape(sc.num_blocks, wl.h_kv, wl.block_size, wl.head_dim, wl.dtype), st)
    keep = set(samp)
    for op in reversed(sc.ops):
        if op[0] == "fork" and op[2] in keep:
            keep.add(op[1])

    def put(seqs, ntok, kv, vv):
        _, slots, pairs = model.append_batch(seqs, ntok)
        if pairs:
            A.copy_blocks(kc, vc, pairs)
        A.write_kv(kc, vc, kv, vv, slots)

    for op in sc.ops:
        kind = op[0]
        if kind == "create" and op[1] in keep:
            model.create(op[1])
        elif kind == "fork" and op[2] in keep:
            model.fork(op[1], op[2])
        elif kind == "free" and op[1] in keep:
            model.free_seq(op[1])
        elif kind == "append" and op[1].seq in keep and op[1].ntok > 0:
            kv, vv = sc.values(op[1])
            put([op[1].seq], op[1].ntok, kv, vv)
        elif kind == "append_rr":
            runs = [r for r in op[1] if r.seq in keep and r.ntok > 0]
            vals = {r.seq: sc.values(r) for r in runs}
            for rr in range(max((r.ntok for r in runs), default=0)):
                live = [r.seq for r in runs if r.ntok > rr]
                put(live, 1, np.stack([vals[q][0][rr] for q in live]),
                    np.stack([vals[q][1][rr] for q in live]))
    tabs = [model.block_table(s) for s in samp]
    maxb = max(len(t) for t, _ in tabs)
    tab = np.full((len(samp), maxb), -1, np.int32)
    lens = np.array([n for _, n in tabs], np.int32)
    for i, (t, _) in enumerate(tabs):
        tab[i, :len(t)] = t
    return kc, vc, tab, lens


def cpu_baseline(sc, budget_s: float, workers: int):
    """Time the oracle (as it stands) on a bounded sample of the same workload.

    Its pool model and cache writes set up the sample (replay_sample); then
    paged_decode over the sample's sequences is repeated until `budget_s`
    seconds have passed.
    The sequences are spread over `workers` forked processes (one BLAS thread
    each), which inherit the sample copy-on-write.  Must run before this
    process touches the GPU: the workers are forked, not started afresh."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    wl = sc.wl
    B = len(sc.decode_seqs)
    nsamp = min(B, max(8, 2 * workers))
    samp = sc.decode_seqs[:nsamp]
    kc, vc, tab, lens = replay_sample(sc, samp)
    kv_bytes = float(lens.sum()) * 2 * wl.h_kv * wl.head_dim * synth.ELEM_BYTES[wl.dtype]
    _SAMPLE.update(q=sc.q[:nsamp], kc=kc, vc=vc, tab=tab, lens=lens, scale=wl.scale,
                   dtype=wl.dtype)
    # longest first, dealt round-robin so the workers get similar work
    order = [int(i) for i in np.argsort(-lens, kind="stable")]
    chunks = [order[w::workers] for w in range(workers) if order[w::workers]]
    reps = 0
    with threadpool_limits(limits=1):
        with mp.get_context("fork").Pool(len(chunks)) as pool:
            pool.map(_oracle_rows, [[r] for r in order[:len(chunks)]])   # workers up
            t0 = time.perf_counter()
            while True:
                done = sum(pool.map(_oracle_rows, chunks, chunksize=1))
                assert done == nsamp
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
            # let the workers finish on their own: leaving the `with` block
            # alone would terminate() them (SIGTERM)
            workers_ = list(pool._pool)
            pool.close()
            pool.join()
    WORKER_EXIT_CODES[:] = [w.exitcode for w in workers_]
    _SAMPLE.clear()
    per_step = el / reps
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       cpu)
    except OSError:
        pass
    return {"value": kv_bytes / per_step / 1e9, "unit": "GB/s", "cores": len(chunks),
            "kind": "oracle", "cpu": cpu,
            "seq_steps_per_s": nsamp / per_step,
            "sample": f"{nsamp} of {B} sequences of {wl.name} (ctx {int(lens.min())}-"
                      f"{int(lens.max())}), fp64 NumPy paged_decode in {len(chunks)} "
                      f"processes x 1 BLAS thread, repeated {reps}x over {el:.1f} s"}


HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_swap(args):
    """Swap half of the workload's sequences out to pinned host blocks and back,
    `steps` times; GB/s of block bytes per direction against the host link."""
    import torch
    import paged_kv_cache_12_amd as pa
    from oracle import attention as A
    from paged_kv_cache_12_amd.manager import PagedKVCache
    wl = synth.WORKLOADS[args.workload or SWAP_WORKLOAD]
    sc = synth.build_scenario(wl)
    dev = torch.device("cuda:0")
    cache = PagedKVCache(sc.num_blocks, wl.block_size, wl.h_kv, wl.head_dim, wl.dtype,
                         device=dev, free_order=sc.free_order)
    fill_cache(sc, cache, dev)
    cache.enable_swap(sc.num_blocks)
    seqs = list(sc.decode_seqs)
    out_set = seqs[: len(seqs) // 2]
    e = synth.ELEM_BYTES[wl.dtype]
    block_bytes = 2 * wl.h_kv * wl.block_size * wl.head_dim * e
    stream = torch.cuda.current_stream()
    for _ in range(2):
        cache.swap_out(out_set)
        cache.swap_in(out_set)
    torch.cuda.synchronize()
    t_out, t_in, host_out, host_in, npairs = [], [], [], [], 0
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        h0 = time.perf_counter()
        pairs = cache.swap_out(out_set)
        h1 = time.perf_counter()
        ev[1].record(stream)
        h2 = time.perf_counter()
        cache.swap_in(out_set)
        h3 = time.perf_counter()
        ev[2].record(stream)
        torch.cuda.synchronize()
        npairs = len(pairs)
        t_out.append(ev[0].elapsed_time(ev[1]))
        t_in.append(ev[1].elapsed_time(ev[2]))
        host_out.append((h1 - h0) * 1e6)
        host_in.append((h3 - h2) * 1e6)
    nbytes = npairs * block_bytes
    # the same bytes as one contiguous copy each way (copy engines)
    flat_d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flat_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    for _ in range(2):
        flat_h.copy_(flat_d, non_blocking=True)
        flat_d.copy_(flat_h, non_blocking=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(5):
        flat_h.copy_(flat_d, non_blocking=True)
    ev[1].record(stream)
    for _ in range(5):
        flat_d.copy_(flat_h, non_blocking=True)
    ev[2].record(stream)
    torch.cuda.synchronize()
    c_out = ev[0].elapsed_time(ev[1]) / 5
    c_in = ev[1].elapsed_time(ev[2]) / 5
    ms_out, ms_in = float(np.mean(t_out)), float(np.mean(t_in))
    # the oracle's swap copy on the host, a bounded sample of the same pairs
    k_np = np.zeros((npairs,) + tuple(cache.k_cache.shape[1:]), synth.STORAGE[wl.dtype])
    v_np = np.zeros_like(k_np)
    kh = np.empty_like(k_np)
    vh = np.empty_like(v_np)
    sample = [(i, i) for i in range(npairs)]
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
        A.swap_blocks(k_np, v_np, kh, vh, sample)
        reps += 1
    cpu_s = (time.perf_counter() - t0) / reps
    res = {
        "metric": "swap of whole sequences to pinned host memory: GB/s of block bytes per "
                  "direction",
        "value": round(nbytes / (ms_out * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "higher_is_better": True, "data": "synthetic",
        "dtype": wl.dtype,
        "config": {"workload": wl.name, "swapped_seqs": len(out_set), "blocks": npairs,
                   "bytes_each_way": nbytes},
        "swap_out_ms": round(ms_out, 4), "swap_in_ms": round(ms_in, 4),
        "swap_in_GBps": round(nbytes / (ms_in * 1e-3) / 1e9, 2),
        "host_us_swap_out_call": round(float(np.median(host_out)), 1),
        "host_us_swap_in_call": round(float(np.median(host_in)), 1),
        "contiguous_copy_GBps": {"d2h": round(nbytes / (c_out * 1e-3) / 1e9, 2),
                                 "h2d": round(nbytes / (c_in * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "host link", "achieved": round(nbytes / (ms_out * 1e-3) / 1e9, 2),
                     "peak": HOST_LINK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (ms_out * 1e-3) / 1e9 / HOST_LINK_GBS, 4),
                     "kernel": "swap_blocks_kernel (device -> pinned host)"},
        "cpu_baseline": {"value": round(nbytes / cpu_s / 1e9, 2), "unit": "GB/s", "cores": 1,
                         "kind": "oracle",
                         "sample": f"oracle swap_blocks over the same {npairs} block pairs in "
                                   f"host memory, repeated {reps}x"},
    }
    print(json.dumps(res), flush=True)


def prefix_stream(seed: int = 105, n_req: int = 256, prefix: int = 4096, bs: int = 16):
    """Requests of the shared-prefix workload as token ids: one 4096-token
    system prompt, then U{64..1024} private tokens per request."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(9,))))
    system = g.integers(0, 32000, prefix).astype(np.int32)
    lens = g.integers(64, 1024, n_req, endpoint=True)
    return [np.concatenate([system, g.integers(0, 32000, int(n)).astype(np.int32)])
            for n in lens]


def bench_prefix(args):
    """Host cost of prefix reuse: every request of the stream through
    pa_seq_create_cached (lookup, allocation, indexing of its new blocks),
    for each index kind; the oracle's model on a bounded sample beside it."""
    import paged_kv_cache_12_amd as pa
    from oracle.pool_model import PoolModel
    bs = 16
    reqs = prefix_stream(bs=bs)
    blocks = sum(-(-len(r) // bs) for r in reqs)
    res = {"metric": "prefix reuse on the host: microseconds per request (create with lookup) "
                     "and hit rate",
           "unit": "us/request", "higher_is_better": False, "data": "synthetic token ids",
           "config": {"workload": "shared 4096-token system prompt + U{64..1024} private tokens",
                      "requests": len(reqs), "block_size": bs,
                      "prompt_tokens": int(sum(len(r) for r in reqs))}}
    # one core's SHA-256 rate: the bound for the hashing index
    buf = np.random.default_rng(0).integers(0, 256, 64 << 20, dtype=np.uint8).tobytes()
    t0 = time.perf_counter()
    pa.sha256(buf)
    sha_gbs = len(buf) / (time.perf_counter() - t0) / 1e9
    for kind, name in ((pa.PA_PREFIX_HASH, "hash"), (pa.PA_PREFIX_RADIX, "radix")):
        per = []
        for rep in range(max(1, min(args.steps, 5))):
            pool = pa.Pool(blocks + 64, bs)
            pool.enable_prefix_cache(kind)
            t0 = time.perf_counter()
            for i, r in enumerate(reqs):
                st, cached, _ = pool.create_cached(i, r)
                assert st == 0
            per.append((time.perf_counter() - t0) / len(reqs) * 1e6)
        stats = pool.prefix_stats()
        us = float(np.median(per))
        res[name] = {"us_per_request": round(us, 2),
                     "hit_rate_blocks": round(stats["hits"] / max(1, stats["queried"]), 4),
                     "cached_tokens_last_request": int(cached),
                     "indexed_blocks": stats["indexed"], "nodes": stats["nodes"]}
        if kind == pa.PA_PREFIX_HASH:
            hashed = sum(len(r) // bs * (bs * 4 + 44) for r in reqs)   # bytes hashed per block
            res[name]["hash_GBps"] = round(hashed / (us * 1e-6 * len(reqs)) / 1e9, 3)
            res[name]["roofline"] = {"bound": "host sha256", "achieved":
                                     res[name]["hash_GBps"], "peak": round(sha_gbs, 3),
                                     "unit": "GB/s", "frac": round(res[name]["hash_GBps"] /
                                                                    sha_gbs, 4)}
    # the oracle's models on the first 16 requests
    sample = reqs[:16]
    cpu = {}
    for kind, name in ((1, "hash"), (2, "radix")):
        m = PoolModel(blocks + 64, bs)
        m.enable_prefix_cache(kind)
        t0 = time.perf_counter()
        for i, r in enumerate(sample):
            m.create_cached(i, r.tolist())
        cpu[name] = round((time.perf_counter() - t0) / len(sample) * 1e6, 1)
    res["value"] = res["hash"]["us_per_request"]
    res["cpu_baseline"] = {"value": cpu["hash"], "unit": "us/request", "cores": 1,
                           "kind": "oracle", "radix_us_per_request": cpu["radix"],
                           "sample": "the oracle's pool model with each index, first 16 "
                                     "requests of the same stream"}
    print(json.dumps(res), flush=True)


def bench_beam(args, width: int = 4):
    """Beam search on the OPT-13B-class shapes (fp16, 40 KV heads, d 128, block
    16): 16 prompts of 1024 tokens, `width` beams each.  One step = one
    pa_beam_decode_step over all beams (each new beam's parent drawn from its
    prompt's beams): pool fork / retire / append, one staging copy,
    pa_copy_blocks of the copy-on-write pairs, pa_write_kv of the new
    positions, pa_decode of all beams."""
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import PagedKVCache
    wl = synth.WORKLOADS["opt13b_sampling_fp16"]
    P, plen, bs = wl.prompts, wl.prompt_len, wl.block_size
    steps_total = args.warmup + args.steps
    need = P * (-(-plen // bs)) + P * width * (steps_total // bs + 2)
    dev = torch.device("cuda:0")
    cache = PagedKVCache(need + 64, bs, wl.h_kv, wl.head_dim, wl.dtype, device=dev)
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    for p in range(P):
        cache.create(p)
        kv = torch.randn((plen, wl.h_kv, wl.head_dim), generator=g, device=dev).half()
        vv = torch.randn((plen, wl.h_kv, wl.head_dim), generator=g, device=dev).half()
        cache.append([p], plen, kv, vv)
    B = P * width
    k_new = torch.randn((B, wl.h_kv, wl.head_dim), generator=g, device=dev).half()
    v_new = torch.randn((B, wl.h_kv, wl.head_dim), generator=g, device=dev).half()
    q = torch.randn((B, wl.h_q, wl.head_dim), generator=g, device=dev).half()
    out = torch.empty_like(q)
    rng = np.random.default_rng(wl.seed)
    maxb = -(-(plen + steps_total + 1) // bs)
    sbytes = pa.pa_decode_step_staging_size(B, maxb)
    h_stage = [torch.empty(sbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    d_stage = torch.empty(sbytes, dtype=torch.uint8, device=dev)
    ws = torch.zeros(max(256, pa.pa_decode_workspace_size(B, wl.h_q, wl.head_dim,
                                                          plen + steps_total + 1, wl.partition),
                         pa.pa_decode_cascade_workspace_size(B, wl.h_q, wl.head_dim,
                                                             plen + steps_total + 1,
                                                             wl.partition)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    done = [None, None]
    beams = [np.arange(P, dtype=np.int64).reshape(P, 1)]   # [prompt][beam] ids
    nxt = [P]
    copies = []
    host_s = []
    nsteps = [0]

    def step():
        # every new beam's parent drawn uniformly from its prompt's beams
        # (one draw for the whole batch)
        cur = beams[0]
        pick = rng.integers(0, cur.shape[1], size=(P, width))
        olds = cur.reshape(-1)
        parents = np.take_along_axis(cur, pick, axis=1).reshape(-1)
        new = np.arange(nxt[0], nxt[0] + P * width, dtype=np.int64).reshape(P, width)
        nxt[0] += P * width
        news = new.reshape(-1)
        beams[0] = new
        j = nsteps[0] & 1
        nsteps[0] += 1
        if done[j] is not None:
            done[j].synchronize()          # staging buffer j is free again
        h0 = time.perf_counter()
        before = cache.pool.stats()["copies"]
        pa.pa_beam_decode_step(cache.pool, olds, parents, news, k_new, v_new, cache.k_cache,
                               cache.v_cache, q, out, wl.scale, wl.partition, maxb, h_stage[j],
                               d_stage, ws)
        host_s.append(time.perf_counter() - h0)
        copies.append(cache.pool.stats()["copies"] - before)
        done[j] = StagingFence(stream)
        return news

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    copies.clear()
    host_s.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        live = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    tab, lens = cache.tables(live)
    e = 2
    logical = float(lens.sum()) * 2 * wl.h_kv * wl.head_dim * e
    unique = unique_kv_bytes(tab, lens, wl)
    block_bytes = 2 * wl.h_kv * bs * wl.head_dim * e
    res = {"metric": "beam-search decode steps: sequence-steps/s (fork, retire, append with "
                     "copy-on-write, block write, decode)",
           "value": round(B / (ms * 1e-3), 1), "unit": "seq-steps/s", "higher_is_better": True,
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": "OPT-13B-class beam search", "prompts": P, "prompt_len": plen,
                      "beam_width": width, "block_size": bs, "partition": wl.partition},
           "cow_pairs_per_step": round(float(np.mean(copies)), 2),
           "cow_bytes_per_step": round(float(np.mean(copies)) * 2 * block_bytes),
           "kv_bytes_logical": round(logical), "kv_bytes_unique": round(unique),
           "effective_unique_GBps": round(unique / (ms * 1e-3) / 1e9, 1),
           "host_us_per_step": round(float(np.median(host_s)) * 1e6, 1)}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU "
              "sharding of this path is design-only.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        calibrate()
        return
    if args.swap:
        bench_swap(args)
        return
    if args.prefix:
        bench_prefix(args)
        return
    if args.beam:
        bench_beam(args)
        return
    workload = args.workload or DEFAULT_WORKLOAD
    also = args.also or (DEFAULT_ALSO if workload == DEFAULT_WORKLOAD else "none")
    names = [workload] + ([also] if also not in ("none", workload) else [])
    scs = {n: synth.build_scenario(synth.WORKLOADS[n]) for n in names}
    # the oracle on the host first: its workers are forked before any GPU use
    cpus = {n: None if args.no_cpu_baseline else
            cpu_baseline(scs[n], args.cpu_seconds, args.cpu_workers or host_cores())
            for n in names}
    res = run_workload(args, scs[names[0]], cpus[names[0]], args.partition)
    for n in names[1:]:
        sub = run_workload(args, scs[n], cpus[n], None)
        res[n] = {k: sub[k] for k in NESTED_KEYS if k in sub}
    print(json.dumps(res), flush=True)


def run_workload(args, sc, cpu, partition):
    """Time `args.steps` steps of one workload (after `args.warmup`), then
    its decode alone, cache cold; returns the JSON record."""
    wl = sc.wl
    part = wl.partition if partition is None else partition
    import torch
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import PagedKVCache, storage_to_torch
    pa.lib()
    dev = torch.device("cuda:0")
    cache = PagedKVCache(sc.num_blocks, wl.block_size, wl.h_kv, wl.head_dim, wl.dtype,
                         device=dev, free_order=sc.free_order)
    fill_cache(sc, cache, dev)
    seqs = np.asarray(sc.decode_seqs, dtype=np.int64)
    B = seqs.size
    e = synth.ELEM_BYTES[wl.dtype]
    total_steps = args.warmup + args.steps
    appends = wl.step_append

    # capacity for the run
    _, lens0 = cache.tables(seqs)
    max_ctx_end = int(lens0.max()) + (total_steps if appends else 0)
    maxb = -(-max_ctx_end // wl.block_size)
    q = storage_to_torch(sc.q, wl.dtype).to(dev)
    out = torch.empty_like(q)
    ws_bytes = max(pa.pa_decode_workspace_size(B, wl.h_q, wl.head_dim, max_ctx_end, part),
                   pa.pa_decode_cascade_workspace_size(B, wl.h_q, wl.head_dim, max_ctx_end, part))
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    step_bytes = []
    host_s = []
    # aliased blocks (forks, shared prefixes): cached loads
    flags = pa.PA_DECODE_SHARED_KV if cache.pool.stats()["shared"] > 0 else 0

    if appends:
        # one native call per step: pool append, one metadata copy, COW copies,
        # block write, decode (pa_decode_step); pinned staging alternates
        step_k = storage_to_torch(sc.step_k, wl.dtype).to(dev)
        step_v = storage_to_torch(sc.step_v, wl.dtype).to(dev)
        sbytes = pa.pa_decode_step_staging_size(B, maxb)
        # four pinned staging buffers in turn and a fence after every second
        # step: before step i refills buffer i % 4, the newest fence recorded
        # after step i - 4 (that of step i - 4 or i - 3) has passed
        h_stage = [torch.empty(sbytes, dtype=torch.uint8, pin_memory=True) for _ in range(4)]
        d_stage = torch.empty(sbytes, dtype=torch.uint8, device=dev)
        fences = {}
        fill = int(lens0.sum())

        def step(i):
            j = i & 3
            if i >= 4:
                k = (i - 4) | 1            # the first fence recorded after step i - 4
                fences[k].synchronize()
                for old in [f for f in fences if f < k]:
                    del fences[old]
            h0 = time.perf_counter()
            pa.pa_decode_step(cache.pool, seqs, step_k, step_v, cache.k_cache, cache.v_cache,
                              q, out, wl.scale, part, maxb, h_stage[j], d_stage, ws)
            host_s.append(time.perf_counter() - h0)
            if i % 2:
                fences[i] = StagingFence(stream)
            step_bytes.append(float(fill + B * (i + 1)) * 2 * wl.h_kv * wl.head_dim * e)
    else:
        tab_h, len_h = cache.tables(seqs, maxb)
        d_tab = torch.from_numpy(tab_h).to(dev)
        d_len = torch.from_numpy(len_h).to(dev)
        max_ctx0 = int(len_h.max())
        kv0 = float(len_h.sum()) * 2 * wl.h_kv * wl.head_dim * e
        order0 = torch.from_numpy(pa.pa_decode_order(tab_h, len_h)).to(dev)
        plan0 = cascade_plan(pa, torch, dev, tab_h, len_h, wl, part, flags)

        def step(i):
            h0 = time.perf_counter()
            run_decode(pa, out, q, cache, d_tab, d_len, max_ctx0, wl, part, ws, flags, order0,
                       plan0)
            host_s.append(time.perf_counter() - h0)
            step_bytes.append(kv0)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kv_step = float(np.mean(step_bytes[args.warmup:]))
    value = kv_step / (ms_step * 1e-3) / 1e9
    hs = np.array(host_s[args.warmup:]) * 1e6
    host_us = {"median": round(float(np.median(hs)), 2),
               "p90": round(float(np.percentile(hs, 90)), 2),
               "what": "host time of the step's native call (pool append, staging, launches)"
               if appends else "host time of the pa_decode call (launch)"}

    # the dominant kernel: pa_decode alone on the final tables, HIP events on
    # its stream.  Cache cold as in a multi-layer decode: the calls cycle
    # through `nrot` copies of the caches (one per layer), so that at least
    # 1 GiB of other KV is read between two reads of one copy (more than the
    # L2s and the MALL hold).  One event pair brackets the timed calls (their
    # average duration); then per-call events (spread) and the same calls on
    # one copy (warm), as diagnostics.
    tab_h, len_h = cache.tables(seqs, maxb)
    d_tab = torch.from_numpy(tab_h).to(dev)
    d_len = torch.from_numpy(len_h).to(dev)
    # the issue order pa_decode_step uses
    d_order = torch.from_numpy(pa.pa_decode_order(tab_h, len_h)).to(dev)
    max_ctx = int(len_h.max())
    kv_dec = float(len_h.sum()) * 2 * wl.h_kv * wl.head_dim * e
    unique = unique_kv_bytes(tab_h, len_h, wl)
    nrot = 1 + math.ceil((1 << 30) / unique)
    copies = [(cache.k_cache, cache.v_cache)] + [
        (cache.k_cache.clone(), cache.v_cache.clone()) for _ in range(nrot - 1)]

    plan = cascade_plan(pa, torch, dev, tab_h, len_h, wl, part, flags)

    def decode(i):
        kc, vc = copies[i % nrot]
        run_decode(pa, out, q, (kc, vc), d_tab, d_len, max_ctx, wl, part, ws, flags, d_order,
                   plan)

    def bracketed(n, rotate):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            decode(i if rotate else 0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(2 * nrot):
        decode(i)
    torch.cuda.synchronize()
    dec_ms = bracketed(args.steps, True)         # average launch duration, cache cold
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a0, a1) in enumerate(evs):
        a0.record(stream)
        decode(i)
        a1.record(stream)
    torch.cuda.synchronize()
    per_call = np.array([a0.elapsed_time(a1) for a0, a1 in evs])
    warm_ms = bracketed(args.steps, False)
    achieved = kv_dec / (dec_ms * 1e-3) / 1e9
    unique_rate = unique / (dec_ms * 1e-3) / 1e9

    # pa_copy_blocks at this workload's shapes: as many pairs as the fill made
    # copy-on-write copies (at least 64), from used blocks into free ones (the
    # decode above never reads a free block), cycling through the copies
    copy = None
    free = cache.pool.free_list()
    used = np.unique(tab_h[tab_h >= 0])
    npairs = min(max(int(cache.pool.stats()["copies"]), 64), free.size, used.size)
    if npairs > 0:
        pairs = np.stack([used[:npairs], free[:npairs]], axis=1).astype(np.int32)
        d_pairs = torch.from_numpy(pairs).to(dev)
        ncopy = 20
        for i in range(nrot):
            pa.pa_copy_blocks(copies[i][0], copies[i][1], d_pairs)
        torch.cuda.synchronize()
        # A copy of a few blocks takes less device time than one launch from
        # Python takes on the host, so the calls are queued behind a spin
        # kernel first: the events then bracket the copies back to back on
        # the device (device time per call, launch gaps on the device
        # included), not the host's launch rate.
        es, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        es.record(stream)
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        h0 = time.perf_counter()
        for i in range(ncopy):
            pa.pa_copy_blocks(copies[i % nrot][0], copies[i % nrot][1], d_pairs)
        queued_s = time.perf_counter() - h0
        e1.record(stream)
        torch.cuda.synchronize()
        c_ms = e0.elapsed_time(e1) / ncopy
        c_bytes = npairs * 2 * 2 * wl.h_kv * wl.block_size * wl.head_dim * e
        copy = {"pairs": npairs, "us_mean": round(c_ms * 1e3, 2),
                "bytes_read_plus_written": c_bytes,
                "GBps": round(c_bytes / (c_ms * 1e-3) / 1e9, 1),
                # true when the spin outlasted the host's queueing of the calls
                "queued_ahead": bool(es.elapsed_time(e0) * 1e-3 > queued_s)}
    del copies
    # context: the same access pattern without the math
    ceiling = read_ceiling(pa, torch, dev, stream)
    ceiling["pattern"] = "random 4 KiB tiles of 4 GiB, 16-byte loads, each tile once (pa_read_probe)"
    ceiling["decode_frac_of_nontemporal"] = round(unique_rate / ceiling["nontemporal_GBps"], 4)

    # HBM bytes per launch from the committed counter runs (rocprofv3 passes
    # of their own over the same command), while the decode code is the one
    # they were taken on
    traffic, traffic_from = None, None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("decode_source_sha256_16") == source_hash() and t.get("partition") == part:
            traffic = t.get("bytes_per_launch")
            traffic_from = os.path.relpath(tfile, ROOT)

    res = {
        "metric": "paged-attn decode: effective KV HBM GB/s (% of peak) + seq-steps/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, no weights)",
        "config": {"workload": wl.name, "batch": B, "q_heads": wl.h_q, "kv_heads": wl.h_kv,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "partition": part,
                   "mean_context": round(kv_dec / (2 * wl.h_kv * wl.head_dim * e) / B, 1),
                   "step": ("append 1 token/seq + " if appends else "") + "decode",
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(B / (ms_step * 1e-3), 1),
        "decode_ms_mean": round(dec_ms, 5),
        "decode_cold_copies": nrot,
        "decode_ms_per_call_p10_median_p90": [round(float(np.percentile(per_call, x)), 5)
                                              for x in (10, 50, 90)],
        "decode_warm_ms_mean": round(warm_ms, 5),
        "warm_achieved": round(unique / (warm_ms * 1e-3) / 1e9, 1),
        "host_us_per_step": host_us,
        "copy_blocks": copy,
        # HBM roofline on the bytes HBM must deliver: each physical block once
        # (equal to the logical bytes unless sequences share blocks)
        "roofline": {"bound": "hbm", "achieved": round(unique_rate, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(unique_rate / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_from": traffic_from,
                     "kernel": "pa_decode" + (" (shared-prefix pass + rest + reduce)"
                                              if plan is not None else
                                              " (partition kernel + reduce)"
                                              if pa.pa_decode_workspace_size(
                                                  B, wl.h_q, wl.head_dim, max_ctx_end, part)
                                              else " (one kernel)"),
                     "cascade_groups": 0 if plan is None else plan["ngroups"],
                     "bytes_per_launch": round(unique),
                     "logical_bytes_per_launch": round(kv_dec),
                     "logical_achieved": round(achieved, 1)},
        "read_ceiling": ceiling,
        "kv_memory": kv_memory(cache.pool.stats()["used"], wl.block_size, unique, kv_dec, len_h,
                               2 * wl.h_kv * wl.head_dim * e),
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    # release this workload's device memory before the next one
    del cache, q, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res




if __name__ == "__main__":
    main()
