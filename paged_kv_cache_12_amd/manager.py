"""Central KV-cache manager: one host block pool plus the device caches.

The vLLM encyclopedia entry (tonho.wtf), section "como funciona", has a single
central KV-cache manager that hands the block tables to the workers together
with each iteration's input.  PagedKVCache is that manager for one GPU: the C++
pool decides slots and copy-on-write pairs, and the device operations
(pa_copy_blocks, pa_write_kv, pa_decode) run on the caller's stream.  Every
metadata tensor of an operation (slots, pairs, tables, lengths, issue order)
is allocated and copied to the device on that same stream, so the kernels
that read it are ordered after its copy, and the caching allocator does not
hand its memory to other work before that stream has passed them.
Whole sequences can be swapped out to pinned host blocks and back (same
entry, "a ideia" and "como funciona").
"""
from __future__ import annotations

import contextlib

import numpy as np

from . import (Pool, PA_OK, PA_DECODE_SHARED_KV, PAError, pa_copy_blocks, pa_decode,
               pa_decode_order, pa_decode_workspace_size, pa_swap_blocks, pa_write_kv)

TORCH_DTYPES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def storage_to_torch(a: np.ndarray, dtype: str):
    """Host storage array (bf16 as uint16 bits) -> CPU torch tensor of dtype."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def torch_to_storage(t, dtype: str) -> np.ndarray:
    """CPU/GPU torch tensor -> host storage array (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class PagedKVCache:
    """Device K/V caches in the library layout plus the host pool.

    guard_blocks extra blocks are allocated before and after the pool proper
    (never handed out) so that tests can check nothing writes outside it.
    """

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype: str, device="cuda", free_order=None, guard_blocks: int = 0,
                 fill_bits: int | None = None):
        import torch
        self.torch = torch
        self.dtype = dtype
        self.tdtype = getattr(torch, TORCH_DTYPES[dtype])
        self.num_blocks, self.bs, self.H, self.d = num_blocks, block_size, num_kv_heads, head_dim
        esz = 4 if dtype == "f32" else 2
        self.x = 16 // esz
        self.guard = guard_blocks
        tot = num_blocks + 2 * guard_blocks
        kshape = (tot, num_kv_heads, head_dim // self.x, block_size, self.x)
        vshape = (tot, num_kv_heads, block_size // self.x, head_dim, self.x)
        self.k_full = torch.empty(kshape, dtype=self.tdtype, device=device)
        self.v_full = torch.empty(vshape, dtype=self.tdtype, device=device)
        if fill_bits is not None:
            ib = torch.int32 if esz == 4 else torch.int16
            val = fill_bits if fill_bits < (1 << (8 * esz - 1)) else fill_bits - (1 << (8 * esz))
            self.k_full.view(ib).fill_(val)
            self.v_full.view(ib).fill_(val)
        self.k_cache = self.k_full[guard_blocks:guard_blocks + num_blocks]
        self.v_cache = self.v_full[guard_blocks:guard_blocks + num_blocks]
        self.pool = Pool(num_blocks, block_size, free_order)
        self.device = device
        self._ws = {}   # decode workspace per stream

    def _on(self, stream):
        """Run the enclosed allocations, copies and launches on `stream` (the
        current stream when None)."""
        if stream is None:
            return contextlib.nullcontext()
        return self.torch.cuda.stream(stream)

    def _to_dev(self, a, dtype):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(self.device)

    # -- pool operations ----------------------------------------------------
    def create(self, seq: int):
        st = self.pool.create(seq)
        if st != PA_OK:
            raise PAError(st, "pa_seq_create")

    def fork(self, parent: int, child: int):
        st = self.pool.fork(parent, child)
        if st != PA_OK:
            raise PAError(st, "pa_seq_fork")

    def free(self, seq: int):
        st = self.pool.free(seq)
        if st != PA_OK:
            raise PAError(st, "pa_seq_free")

    # -- swapping to pinned host memory -----------------------------------------
    def enable_swap(self, num_host_blocks: int):
        """Pinned host caches of num_host_blocks blocks (same layout) and the
        pool's host block ids."""
        torch = self.torch
        kshape = (num_host_blocks,) + tuple(self.k_cache.shape[1:])
        vshape = (num_host_blocks,) + tuple(self.v_cache.shape[1:])
        self.k_host = torch.empty(kshape, dtype=self.tdtype, pin_memory=True)
        self.v_host = torch.empty(vshape, dtype=self.tdtype, pin_memory=True)
        st = self.pool.set_host_blocks(num_host_blocks)
        if st != PA_OK:
            raise PAError(st, "pa_pool_set_host_blocks")

    def _pairs_to_device(self, pairs):
        # through pinned memory, so the host does not wait for earlier work on
        # the (current) stream
        t = self.torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).pin_memory()
        return t.to(self.device, non_blocking=True)

    def swap_out(self, seqs, stream=None):
        """Move seqs (all or none) to host blocks; the device -> host copies run
        on `stream`.  Returns the (gpu, host) pairs."""
        st, pairs = self.pool.swap_out(np.asarray(seqs, dtype=np.int64))
        if st != PA_OK:
            raise PAError(st, "pa_seq_swap_out")
        if len(pairs):
            with self._on(stream):
                pa_swap_blocks(self.k_cache, self.v_cache, self.k_host, self.v_host,
                               self._pairs_to_device(pairs))
        return pairs

    def swap_in(self, seqs, stream=None):
        """Bring swapped seqs back (all or none); host -> device copies on
        `stream`.  Returns the (host, gpu) pairs."""
        st, pairs = self.pool.swap_in(np.asarray(seqs, dtype=np.int64))
        if st != PA_OK:
            raise PAError(st, "pa_seq_swap_in")
        if len(pairs):
            with self._on(stream):
                pa_swap_blocks(self.k_host, self.v_host, self.k_cache, self.v_cache,
                               self._pairs_to_device(pairs))
        return pairs

    # -- prefix reuse -----------------------------------------------------------------
    def enable_prefix_cache(self, kind: int):
        st = self.pool.enable_prefix_cache(kind)
        if st != PA_OK:
            raise PAError(st, "pa_pool_enable_prefix_cache")

    def create_cached(self, seq: int, tokens, k_of, v_of, salt: bytes = b"",
                      extra: bytes = b"", stream=None):
        """New sequence for prompt `tokens` through the prefix index; only the
        positions not found in it are written: k_of(start, end) / v_of(start,
        end) give their K/V as GPU tensors [end-start][H_kv][d].  Returns the
        number of cached tokens."""
        st, cached, slots = self.pool.create_cached(seq, tokens, salt, extra)
        if st != PA_OK:
            raise PAError(st, "pa_seq_create_cached")
        n = len(tokens)
        if n > cached:
            with self._on(stream):
                pa_write_kv(k_of(cached, n), v_of(cached, n), self.k_cache, self.v_cache,
                            self._to_dev(slots, np.int64))
        return cached

    def append_tokens(self, seqs, tokens, k_new, v_new, stream=None):
        """append() with token ids [len(seqs)][k], so the prefix index keeps
        indexing the blocks these sequences fill."""
        st, slots, pairs = self.pool.append_tokens(np.asarray(seqs, dtype=np.int64), tokens)
        if st != PA_OK:
            raise PAError(st, "pa_seq_append_tokens")
        self._copy_and_write(pairs, slots, k_new, v_new, stream)
        return slots, pairs

    # -- beam search ----------------------------------------------------------------
    def beam_step(self, old_beams, parents, new_beams, k_new, v_new, tokens=None, stream=None):
        """One beam-search step: new beams fork their parents, old beams retire,
        each new beam gets one position (k_new / v_new [len(new_beams)][H][d]);
        the copy-on-write copies run before the block write."""
        st, slots, pairs = self.pool.beam_step(old_beams, parents, new_beams, tokens)
        if st != PA_OK:
            raise PAError(st, "pa_seq_beam_step")
        self._copy_and_write(pairs, slots, k_new, v_new, stream)
        return slots, pairs

    def _copy_and_write(self, pairs, slots, k_new, v_new, stream):
        """Copy-on-write copies, then the block write, with their metadata, on
        `stream`."""
        with self._on(stream):
            if len(pairs):
                pa_copy_blocks(self.k_cache, self.v_cache, self._to_dev(pairs, np.int32))
            if len(slots):
                pa_write_kv(k_new, v_new, self.k_cache, self.v_cache,
                            self._to_dev(slots, np.int64))

    # -- append: pool slots, copy-on-write, block write ----------------------
    def append(self, seqs, k: int, k_new, v_new, stream=None):
        """Append k tokens to each sequence in `seqs` (in order).  k_new, v_new:
        GPU tensors [len(seqs)*k][H][d] in the same order.  Runs pa_copy_blocks
        for any copy-on-write pair before pa_write_kv.  Returns (slots, pairs)."""
        st, slots, pairs = self.pool.append_batch(seqs, k)
        if st != PA_OK:
            raise PAError(st, "pa_seq_append_batch")
        self._copy_and_write(pairs, slots, k_new, v_new, stream)
        return slots, pairs

    # -- decode ---------------------------------------------------------------
    def tables(self, seqs, maxb: int | None = None):
        """Host block tables [n][maxb] (-1 padded) and context lengths."""
        seqs = np.asarray(seqs, dtype=np.int64)
        if maxb is None:
            maxb = 1
            for s in seqs:
                t, _ = self.pool.block_table(int(s))
                maxb = max(maxb, len(t))
        return self.pool.block_tables(seqs, maxb)

    def decode(self, q, seqs, scale: float, partition_size: int = 512, out=None, stream=None):
        """Decode attention of q [len(seqs)][H_q][d] over the sequences' blocks
        on `stream`.  The workspace is kept per stream: decodes on one stream
        reuse it in stream order."""
        torch = self.torch
        tables, lens = self.tables(seqs)
        max_ctx = int(lens.max()) if lens.size else 0
        flags = PA_DECODE_SHARED_KV if self.pool.stats()["shared"] > 0 else 0
        order = pa_decode_order(tables, lens)
        with self._on(stream):
            cur = torch.cuda.current_stream(self.device)
            bt = self._to_dev(tables, np.int32)
            ln = self._to_dev(lens, np.int32)
            d_order = self._to_dev(order, np.int32)
            if out is None:
                out = torch.empty_like(q)
            need = pa_decode_workspace_size(q.shape[0], q.shape[1], self.d, max_ctx,
                                            partition_size)
            ws = self._ws.get(cur.cuda_stream)
            if need and (ws is None or ws.numel() < need):
                ws = torch.empty(need, dtype=torch.uint8, device=self.device)
                self._ws[cur.cuda_stream] = ws
            pa_decode(out, q, self.k_cache, self.v_cache, bt, ln, max_ctx, scale,
                      partition_size, workspace=ws if need else None, flags=flags,
                      seq_order=d_order)
        return out, tables, lens
