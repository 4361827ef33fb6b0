"""fp64 reference for PagedAttention decode (test infrastructure only).

What is computed.  The vLLM encyclopedia entry (tonho.wtf), section "como
funciona", describes decode attention rewritten block by block: the current
token's query is multiplied by the keys of one KV block at a time, giving that
slice of the score vector, and the output is accumulated against the values of
the same block; blocks need not be adjacent in memory.  All three explainers
("PagedAttention e RadixAttention, parliamo di KV Cache", section "PagedAttention:
la memoria come un sistema operativo"; "LLM : PagedAttention et RadixAttention
optimisent le cache KV", section "PagedAttention traite la mémoire"; "KV Cache
Administration", section "Why this modified LLM serving") state that paging
changes neither the attention algorithm nor the model outputs.  So the oracle
is plain contiguous attention: rebuild each sequence's K and V in logical token
order through its block table, then softmax(q K^T * scale) V in float64.

Readings where the pages are silent:
  * scale = 1/sqrt(head_dim), passed in by the caller;
  * grouped-query attention (the same entry, section "onde isso aparece hoje",
    names K/V shared between heads): query head h reads KV head h // G with
    G = H_q / H_kv (contiguous groups);
  * a sequence with zero context produces a zero output row.

Cache layout (the library's ABI; the pages do not fix one).  With
x = 16 / element_bytes (8 for fp16/bf16, 4 for fp32):
  K cache [num_blocks][H_kv][head_dim/x][block_size][x]:
      element (block b, head h, token-in-block t, dim i) at
      [b][h][i//x][k_row(t)][i%x], where k_row stores the tokens whose index
      has bit 2 clear first (in increasing order), then those with bit 2 set
  V cache [num_blocks][H_kv][block_size/x][head_dim][x]:
      element (b, h, t, i) at [b][h][t//x][i][t%x]
"""
from __future__ import annotations

import math

import numpy as np

_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def vec_elems(dtype: str) -> int:
    """x: elements per 16-byte vector."""
    return 16 // _ELEM_BYTES[dtype]


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64 (bf16 is stored as uint16 bits)."""
    if dtype in ("f32", "f16"):
        return raw.astype(np.float64)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Cache layout: explicit per-element offsets, and whole-array views.
# ----------------------------------------------------------------------------

def k_row(t, bs):
    """Row of token t inside a K slab: tokens with bit 2 clear, then set."""
    return (bs // 2 if t & 4 else 0) + 4 * (t >> 3) + (t & 3)


def k_offset(b, h, t, i, H, bs, d, x):
    """Flat element offset of K(block b, head h, token t, dim i)."""
    return (((b * H + h) * (d // x) + i // x) * bs + k_row(t, bs)) * x + i % x


def v_offset(b, h, t, i, H, bs, d, x):
    """Flat element offset of V(block b, head h, token t, dim i)."""
    return (((b * H + h) * (bs // x) + t // x) * d + i) * x + t % x


def k_cache_shape(num_blocks, H, bs, d, dtype):
    x = vec_elems(dtype)
    return (num_blocks, H, d // x, bs, x)


def v_cache_shape(num_blocks, H, bs, d, dtype):
    x = vec_elems(dtype)
    return (num_blocks, H, bs // x, d, x)


def _k_rows(bs):
    return np.array([k_row(t, bs) for t in range(bs)], dtype=np.int64)


def _k_tokens(kblocks: np.ndarray) -> np.ndarray:
    """[n][H][d/x][bs rows][x] -> [n*bs][H][d] in logical token order."""
    n, H, dx, bs, x = kblocks.shape
    by_token = kblocks[:, :, :, _k_rows(bs), :]
    return by_token.transpose(0, 3, 1, 2, 4).reshape(n * bs, H, dx * x)


def _v_tokens(vblocks: np.ndarray) -> np.ndarray:
    """[n][H][bs/x][d][x] -> [n*bs][H][d] in logical token order."""
    n, H, bx, d, x = vblocks.shape
    return vblocks.transpose(0, 2, 4, 1, 3).reshape(n * bx * x, H, d)


def gather_sequence(k_cache, v_cache, table, ctx: int, dtype: str):
    """Contiguous K, V [ctx][H_kv][d] (float64) of one sequence.

    Only the first ceil(ctx / block_size) table entries are read; the rest of
    the table and the unfilled tail of the last block are never touched.
    """
    bs = k_cache.shape[3]
    nb = -(-ctx // bs)
    blocks = np.asarray(table[:nb], dtype=np.int64)
    if nb and (blocks.min() < 0 or blocks.max() >= k_cache.shape[0]):
        raise ValueError("block table entry out of range")
    K = _k_tokens(k_cache[blocks])[:ctx]
    V = _v_tokens(v_cache[blocks])[:ctx]
    return to_f64(K, dtype), to_f64(V, dtype)


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def attention_contiguous(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                         return_p: bool = False):
    """q [H_q][d], K/V [n][H_kv][d] (float64) -> out [H_q][d].

    out[h] = softmax(K[:, h//G] @ q[h] * scale) @ V[:, h//G].
    """
    H_q, d = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((H_q, d), dtype=np.float64)
    P = np.zeros((H_q, n), dtype=np.float64)
    if n == 0:
        return (out, P) if return_p else out
    for h in range(H_q):
        kv = h // G
        z = (K[:, kv, :] @ q[h]) * scale
        w = np.exp(z - z.max())
        p = w / w.sum()
        out[h] = p @ V[:, kv, :]
        P[h] = p
    return (out, P) if return_p else out


def paged_decode(q_raw, k_cache, v_cache, block_tables, ctx_lens, scale: float,
                 dtype: str, seqs=None):
    """Decode attention for a batch.  q_raw [B][H_q][d] in storage format;
    block_tables [B][maxb] int; ctx_lens [B] int.  Returns float64 [B][H_q][d]
    (only the rows listed in `seqs`, if given, are computed; others are NaN)."""
    q = to_f64(np.asarray(q_raw), dtype)
    B, H_q, d = q.shape
    out = np.full((B, H_q, d), np.nan)
    for s in (range(B) if seqs is None else seqs):
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], int(ctx_lens[s]), dtype)
        out[s] = attention_contiguous(q[s], K, V, scale)
    return out


def split_attention(q, K, V, scale: float, partition: int):
    """Split-K form: partitions [p*P, p*P+P) of the context each give
    (m_p, l_p, o_p) = (max score, sum of exp(score - m_p), unnormalised output);
    they are combined with M = max m_p, L = sum e^(m_p - M) l_p,
    out = sum e^(m_p - M) o_p / L, in ascending p.  Mathematically identical to
    attention_contiguous."""
    H_q, d = q.shape
    n, H_kv, _ = K.shape
    G = H_q // H_kv
    out = np.zeros((H_q, d))
    if n == 0:
        return out
    nparts = -(-n // partition)
    for h in range(H_q):
        kv = h // G
        ms, ls, os_ = [], [], []
        for p in range(nparts):
            lo, hi = p * partition, min(n, (p + 1) * partition)
            z = (K[lo:hi, kv, :] @ q[h]) * scale
            m = z.max()
            w = np.exp(z - m)
            ms.append(m)
            ls.append(w.sum())
            os_.append(w @ V[lo:hi, kv, :])
        M = max(ms)
        L = sum(math.exp(m - M) * l for m, l in zip(ms, ls))
        acc = np.zeros(d)
        for m, o in zip(ms, os_):
            acc += math.exp(m - M) * o
        out[h] = acc / L
    return out


# ----------------------------------------------------------------------------
# Data movement: block write and block copy
# ----------------------------------------------------------------------------

def write_kv(k_cache, v_cache, k_new, v_new, slots):
    """Store token j's K/V [H_kv][d] at slot = block*bs + offset; slots < 0 are
    skipped.  In-place on the (storage-format) cache arrays."""
    nbk, H, dx, bs, x = k_cache.shape
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    s = slots[keep]
    b, t = s // bs, s % bs
    kn = np.asarray(k_new)[keep]          # [T][H][d]
    vn = np.asarray(v_new)[keep]
    T = kn.shape[0]
    d = kn.shape[2]
    # K: [b][h][i//x][k_row(t)][i%x] <- kn[j][h][i]
    k_cache[b, :, :, _k_rows(bs)[t], :] = kn.reshape(T, H, d // x, x)
    # V: [b][h][t//x][i][t%x] <- vn[j][h][i]
    v_cache[b, :, t // x, :, t % x] = vn


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Swap copies between a GPU cache and a host cache (tonho.wtf, "a ideia":
    swap to CPU RAM): for each (src, dst) pair the whole block of K and of V
    moves from the source cache to the destination cache."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def copy_blocks(k_cache, v_cache, pairs):
    """For each (src, dst) pair in order, copy the whole physical block (all
    heads, all positions) of K and of V."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]
