"""Seeded synthetic inputs for PagedAttention decode workloads.

This module only draws random numbers and lays out *what happens* in a
workload: sequence lengths, the pool's free order, the script of pool
operations (create / fork / append / free), per-token K/V values in logical
token order, queries and the new K/V of a decode step.  It holds none of the
method's arithmetic: no slot mapping, no cache layout, no attention.  Both the
oracle-side tests and the GPU-side tests and bench consume it.

Values are float32 N(0,1) draws rounded to the workload's dtype (RNE).
Storage convention for raw arrays: float32 -> np.float32, fp16 -> np.float16,
bf16 -> np.uint16 holding the bf16 bit pattern.

Every array is keyed by (seed, stream, key, chunk) through numpy's
SeedSequence spawn keys, so the values do not depend on how many threads
produced them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

_CHUNK_TOKENS = 4096
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# Streams: distinct spawn-key prefixes for independent draws.
_S_K, _S_V, _S_Q, _S_STEP_K, _S_STEP_V = 1, 2, 3, 4, 5


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Inputs here are finite N(0,1) draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def cast_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def _gen(seed: int, key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def normal_array(seed: int, key: tuple, shape: tuple, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws of `shape`, rounded to dtype storage."""
    g = _gen(seed, key)
    return cast_storage(g.standard_normal(shape, dtype=np.float32), dtype)


def token_values(seed: int, stream: int, key: int, ntok: int, heads: int, dim: int,
                 dtype: str) -> np.ndarray:
    """[ntok][heads][dim] values for one run of tokens, chunked by 4096 tokens."""
    out = np.empty((ntok, heads, dim), dtype=STORAGE[dtype])
    nchunks = (ntok + _CHUNK_TOKENS - 1) // _CHUNK_TOKENS

    def work(c):
        lo = c * _CHUNK_TOKENS
        hi = min(ntok, lo + _CHUNK_TOKENS)
        out[lo:hi] = normal_array(seed, (stream, key, c), (hi - lo, heads, dim), dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nchunks)))
    return out


# ----------------------------------------------------------------------------
# Workload definitions (shapes only; no weights are involved)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    batch: int
    h_q: int
    h_kv: int
    head_dim: int
    block_size: int
    seed: int
    partition: int = 512
    ctx_lo: int = 1
    ctx_hi: int = 1
    pool_blocks: int = 0          # 0 -> 1.25x what the script needs
    kind: str = "plain"           # plain | sampling | prefix
    # sampling (parallel sampling): prompts, samples per prompt, private tokens
    prompts: int = 0
    samples: int = 0
    prompt_len: int = 0
    gen_hi: int = 0
    cow: bool = False             # prompt lengths 1024 - r, r ~ U{1..15}
    # shared prefix
    prefix_len: int = 0
    step_append: bool = False     # each decode step appends one token per sequence
    description: str = ""

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    "tiny_mha_fp32": Workload(
        name="tiny_mha_fp32", dtype="f32", batch=4, h_q=4, h_kv=4, head_dim=64,
        block_size=16, seed=101, ctx_lo=1, ctx_hi=200, pool_blocks=64,
        description="1 layer, batch 4, 4 heads (MHA), d 64, bs 16, ctx U[1,200], pool 64"),
    "llama3_8b_gqa_bf16": Workload(
        name="llama3_8b_gqa_bf16", dtype="bf16", batch=64, h_q=32, h_kv=8, head_dim=128,
        block_size=16, seed=102, ctx_lo=512, ctx_hi=4096, step_append=True, partition=0,
        description="Llama-3-8B-class layer: 32 q / 8 kv heads, d 128, bs 16, batch 64, "
                    "ctx U[512,4096] + one appended token per step"),
    "opt13b_sampling_fp16": Workload(
        name="opt13b_sampling_fp16", dtype="f16", batch=64, h_q=40, h_kv=40, head_dim=128,
        block_size=16, seed=103, kind="sampling", prompts=16, samples=4, prompt_len=1024,
        gen_hi=1024,
        description="OPT-13B-class MHA: 40 heads, d 128, bs 16, 16 prompts x 4 samples, "
                    "prompt 1024, private tokens U[0,1024]"),
    "opt13b_sampling_cow_fp16": Workload(
        name="opt13b_sampling_cow_fp16", dtype="f16", batch=64, h_q=40, h_kv=40, head_dim=128,
        block_size=16, seed=103, kind="sampling", prompts=16, samples=4, prompt_len=1024,
        gen_hi=1024, cow=True,
        description="as opt13b_sampling_fp16 but prompt lengths 1024-r, r~U{1..15}, so the "
                    "shared last prompt block is partly filled and appends copy it"),
    "long_70b_gqa_bf16": Workload(
        name="long_70b_gqa_bf16", dtype="bf16", batch=8, h_q=64, h_kv=8, head_dim=128,
        block_size=32, seed=104, ctx_lo=32768, ctx_hi=131072, partition=512,
        step_append=True,
        description="70B-class layer: 64 q / 8 kv heads, d 128, bs 32, batch 8, "
                    "ctx U[32768,131072] + one appended token per step, 512-token "
                    "split-K partitions"),
    "shared_prefix_bf16": Workload(
        name="shared_prefix_bf16", dtype="bf16", batch=256, h_q=32, h_kv=8, head_dim=128,
        block_size=16, seed=105, kind="prefix", prefix_len=4096, ctx_lo=64, ctx_hi=1024,
        description="256 sequences aliasing one 4096-token prefix (256 blocks of 16) plus "
                    "private suffixes U[64,1024]; 32 q / 8 kv heads, d 128"),
}


# ----------------------------------------------------------------------------
# Scenario: the op script plus values
# ----------------------------------------------------------------------------

@dataclass
class Run:
    """A run of `ntok` tokens appended to `seq`; values come from
    token_values(seed, stream, key, ...)."""
    seq: int
    ntok: int
    key: int


@dataclass
class Scenario:
    wl: Workload
    num_blocks: int
    free_order: np.ndarray                  # int32 permutation of [0, num_blocks)
    ops: list                               # ("create", s) | ("fork", p, c) | ("free", s)
                                            # | ("append", Run) | ("append_rr", [Run...])
    decode_seqs: list                       # batch order of the decode step
    q: np.ndarray                           # [B][H_q][d] storage
    step_k: np.ndarray | None = None        # [B][H_kv][d] storage (step_append)
    step_v: np.ndarray | None = None
    lengths: dict = field(default_factory=dict)  # drawn lengths, for reporting

    def values(self, run: Run):
        wl = self.wl
        k = token_values(wl.seed, _S_K, run.key, run.ntok, wl.h_kv, wl.head_dim, wl.dtype)
        v = token_values(wl.seed, _S_V, run.key, run.ntok, wl.h_kv, wl.head_dim, wl.dtype)
        return k, v


def prefix_values(tokens, start: int, end: int, heads: int, dim: int, dtype: str,
                  seed: int = 0):
    """K and V [end-start][heads][dim] for positions start..end-1 of a token
    list, each drawn from a generator seeded by the token ids up to and
    including that position (a rolling SHA-256), so equal prefixes give equal
    values wherever they occur, as a model's K/V would."""
    import hashlib
    h = hashlib.sha256(seed.to_bytes(8, "little")).digest()
    kv = np.empty((2, end - start, heads, dim), dtype=np.float32)
    for pos in range(end):
        h = hashlib.sha256(h + int(tokens[pos]).to_bytes(4, "little", signed=True)).digest()
        if pos >= start:
            g = np.random.Generator(np.random.PCG64(int.from_bytes(h[:8], "little")))
            kv[:, pos - start] = g.standard_normal((2, heads, dim), dtype=np.float32)
    return cast_storage(kv[0], dtype), cast_storage(kv[1], dtype)


def _ceil_div(a, b):
    return -(-a // b)


def build_scenario(wl: Workload, batch: int | None = None, ctx_hi: int | None = None,
                   samples_override: int | None = None) -> Scenario:
    """Draw the workload.  `batch` / `ctx_hi` shrink it for fast tests while
    keeping the same structure (the draws then differ from the full size)."""
    g = _gen(wl.seed, (0,))
    bs = wl.block_size
    ops: list = []
    lengths: dict = {}
    B = batch if batch is not None else wl.batch
    hi = ctx_hi if ctx_hi is not None else wl.ctx_hi

    if wl.kind == "plain":
        lens = g.integers(wl.ctx_lo, hi, size=B, endpoint=True)
        lengths["ctx"] = lens
        extra = 1 if wl.step_append else 0
        need = int(sum(_ceil_div(int(n) + extra, bs) for n in lens))
        nblocks = wl.pool_blocks or int(math.ceil(1.25 * need))
        free_order = g.permutation(nblocks).astype(np.int32)
        for s in range(B):
            ops.append(("create", s))
            ops.append(("append", Run(s, int(lens[s]), s)))
        decode = list(range(B))
    elif wl.kind == "sampling":
        P = B // wl.samples if batch is not None else wl.prompts
        S = wl.samples
        if wl.cow:
            r = g.integers(1, 15, size=P, endpoint=True)
        else:
            r = np.zeros(P, dtype=np.int64)
        plen = wl.prompt_len - r
        gen_hi = hi if ctx_hi is not None else wl.gen_hi
        gens = g.integers(0, gen_hi, size=P * S, endpoint=True)
        lengths["prompt"] = plen
        lengths["gen"] = gens
        need = int(sum(_ceil_div(int(n), bs) for n in plen))
        need += int(sum(_ceil_div(int(x), bs) + 1 for x in gens))
        nblocks = wl.pool_blocks or int(math.ceil(1.25 * need))
        free_order = g.permutation(nblocks).astype(np.int32)
        key = 0
        for p in range(P):
            parent = p * S
            ops.append(("create", parent))
            ops.append(("append", Run(parent, int(plen[p]), key)))
            key += 1
            for j in range(1, S):
                ops.append(("fork", parent, parent + j))
        # private tokens, appended round-robin one token per live sample per round
        runs = [Run(s, int(gens[s]), key + s) for s in range(P * S)]
        ops.append(("append_rr", runs))
        decode = list(range(P * S))
    elif wl.kind == "prefix":
        sfx = g.integers(wl.ctx_lo, hi, size=B, endpoint=True)
        lengths["suffix"] = sfx
        need = _ceil_div(wl.prefix_len, bs) + int(sum(_ceil_div(int(x), bs) + 1 for x in sfx))
        nblocks = wl.pool_blocks or int(math.ceil(1.25 * need))
        free_order = g.permutation(nblocks).astype(np.int32)
        tmpl = B  # template sequence id, freed after the forks
        ops.append(("create", tmpl))
        ops.append(("append", Run(tmpl, wl.prefix_len, 0)))
        for s in range(B):
            ops.append(("fork", tmpl, s))
        ops.append(("free", tmpl))
        for s in range(B):
            ops.append(("append", Run(s, int(sfx[s]), 1 + s)))
        decode = list(range(B))
    else:
        raise ValueError(wl.kind)

    nb = len(decode)
    q = normal_array(wl.seed, (_S_Q,), (nb, wl.h_q, wl.head_dim), wl.dtype)
    sk = sv = None
    if wl.step_append:
        sk = normal_array(wl.seed, (_S_STEP_K,), (nb, wl.h_kv, wl.head_dim), wl.dtype)
        sv = normal_array(wl.seed, (_S_STEP_V,), (nb, wl.h_kv, wl.head_dim), wl.dtype)
    return Scenario(wl=wl, num_blocks=nblocks, free_order=free_order, ops=ops,
                    decode_seqs=decode, q=q, step_k=sk, step_v=sv, lengths=lengths)


def poison_bits(dtype: str) -> int:
    """A quiet-NaN bit pattern used to fill never-written cache slots."""
    return {"f32": 0x7FC0DEAD, "f16": 0x7E5A, "bf16": 0x7FDA}[dtype]
