"""Python binding of libpa.so (PagedAttention decode for MI355X / gfx950).

Argument marshalling only: every step of the decode path runs in libpa.so's
HIP kernels or its C++ host pool.  Device arrays are torch tensors on the GPU
(torch is used for device memory and streams); host arrays are numpy arrays.
The functions keep the C names: pa_write_kv, pa_copy_blocks, pa_decode,
pa_decode_workspace_size, and the pool wrapper `Pool` over pa_pool_* /
pa_seq_*.  If libpa.so is missing every call raises; there is no fallback.

Cache tensors have the library layout (x = 16 / element bytes):
  K [num_blocks][H_kv][head_dim/x][block_size][x]
  V [num_blocks][H_kv][block_size/x][head_dim][x]
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libpa.so")

(PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_NO_BLOCKS, PA_ERR_UNKNOWN_SEQ, PA_ERR_HIP,
 PA_ERR_TOO_LARGE) = range(7)
PA_NOALLOC_SCRATCH_BYTES = 64 << 20
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_DECODE_SHARED_KV = 1
PA_PREFIX_HASH, PA_PREFIX_RADIX = 1, 2
DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16}

# name -> (restype, argtypes), mirroring include/pa.h
_c = ctypes
_vp, _i, _i64, _f, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t
SIGNATURES = {
    "pa_status_str": (_c.c_char_p, [_i]),
    "pa_abi_version": (_i, []),
    "pa_write_kv": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "pa_copy_blocks": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "pa_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "pa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                       _i, _vp, _sz, _i, _i, _vp]),
    "pa_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i,
                               _i, _f, _i, _i, _i, _vp]),
    "pa_decode_order": (_i, [_vp, _i, _vp, _i, _vp]),
    "pa_cascade_plan": (_i, [_vp, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp]),
    "pa_decode_cascade_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "pa_decode_cascade": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                               _f, _i, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _i, _i, _vp]),
    "pa_swap_blocks": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _vp]),
    "pa_read_probe_partials": (_i, []),
    "pa_read_probe": (_i, [_vp, _i64, _i, _vp, _i, _vp, _vp]),
    "pa_pool_set_host_blocks": (_i, [_vp, _i]),
    "pa_seq_swap_out": (_i, [_vp, _vp, _i, _vp, _i, _vp]),
    "pa_seq_swap_in": (_i, [_vp, _vp, _i, _vp, _i, _vp]),
    "pa_seq_is_swapped": (_i, [_vp, _i64]),
    "pa_pool_host_stats": (_i, [_vp, _vp]),
    "pa_sha256": (_i, [_vp, _sz, _vp]),
    "pa_prefix_block_hash": (_i, [_vp, _vp, _i, _vp, _i, _vp]),
    "pa_pool_enable_prefix_cache": (_i, [_vp, _i]),
    "pa_seq_create_cached": (_i, [_vp, _i64, _vp, _i, _vp, _i, _vp, _i, _vp, _vp]),
    "pa_seq_append_tokens": (_i, [_vp, _vp, _i, _vp, _i, _vp, _vp, _vp]),
    "pa_prefix_stats": (_i, [_vp, _vp]),
    "pa_seq_beam_step": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp]),
    "pa_beam_decode_step": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                 _i, _vp, _vp, _i, _f, _i, _i, _vp, _vp, _sz, _vp, _sz, _i, _vp]),
    "pa_decode_step_staging_size": (_sz, [_i, _i]),
    "pa_decode_step": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _i,
                            _f, _i, _i, _vp, _vp, _sz, _vp, _sz, _i, _vp]),
    "pa_pool_create": (_i, [_i, _i, _vp, _c.POINTER(_vp)]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_seq_create": (_i, [_vp, _i64]),
    "pa_seq_fork": (_i, [_vp, _i64, _i64]),
    "pa_seq_append": (_i, [_vp, _i64, _i, _vp, _vp, _vp]),
    "pa_seq_append_batch": (_i, [_vp, _vp, _i, _i, _vp, _vp, _vp]),
    "pa_seq_free": (_i, [_vp, _i64]),
    "pa_seq_block_table": (_i, [_vp, _i64, _vp, _i, _vp, _vp]),
    "pa_pool_block_tables": (_i, [_vp, _vp, _i, _vp, _i, _vp]),
    "pa_pool_refcount": (_i, [_vp, _c.c_int32]),
    "pa_pool_free_list": (_i, [_vp, _vp, _i, _vp]),
    "pa_pool_stats": (_i, [_vp, _vp]),
    "pa_kv_bytes_per_token": (_sz, [_i, _i, _i, _i]),
}

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    """Load libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_12_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    try:
        return lib().pa_status_str(status).decode()
    except Exception:
        return "?"


def _check(status: int, what: str):
    if status != PA_OK:
        raise PAError(status, what)


# ----------------------------------------------------------------------------
# torch marshalling helpers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev_ptr(t, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() or None


def _any_ptr(t, name: str) -> int:
    """GPU tensor or pinned CPU tensor (device-reachable memory)."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
    return t.data_ptr()


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def cache_geometry(k_cache, v_cache):
    """(num_blocks, H_kv, block_size, head_dim) from cache tensors."""
    if k_cache.dim() != 5 or v_cache.dim() != 5:
        raise ValueError("cache tensors must be 5-d (library layout)")
    nb, H, dx, bs, x = k_cache.shape
    nb2, H2, bx, d, x2 = v_cache.shape
    if (nb, H, x) != (nb2, H2, x2) or dx * x != d or bx * x != bs:
        raise ValueError("K and V cache shapes disagree")
    if k_cache.dtype != v_cache.dtype or k_cache.element_size() * x != 16:
        raise ValueError("cache dtype / vector width mismatch")
    return nb, H, bs, d


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_same_dtype(ref, **tensors):
    for name, t in tensors.items():
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, the cache is {ref.dtype}")


def _check_decode_io(out, q, k_cache, v_cache):
    """Shapes and dtypes of a decode's q / out against the cache; returns
    (num_blocks, H_kv, block_size, head_dim, B, H_q).  Every check runs before
    any pointer is taken, so a mismatch never reaches a kernel."""
    nb, H_kv, bs, d = cache_geometry(k_cache, v_cache)
    torch_dtype_code(k_cache)
    _check_same_dtype(k_cache, q=q, out=out)
    if q.dim() != 3 or q.shape[2] != d:
        raise ValueError(f"q must be [num_seqs][num_q_heads][{d}], got {tuple(q.shape)}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out shape {tuple(out.shape)} != q shape {tuple(q.shape)}")
    B, H_q, _ = q.shape
    if H_q % H_kv != 0:
        raise ValueError(f"num_q_heads {H_q} is not a multiple of num_kv_heads {H_kv}")
    return nb, H_kv, bs, d, B, H_q


def _check_tables(block_tables, context_lens, B):
    torch = _torch()
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables / context_lens shape mismatch")


def _check_new_kv(k_new, v_new, k_cache, n, H_kv, d):
    _check_same_dtype(k_cache, k_new=k_new, v_new=v_new)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (n, H_kv, d):
            raise ValueError(f"{name} must be [{n}][{H_kv}][{d}], got {tuple(t.shape)}")


def _seq_ids(seqs, name: str = "seqs") -> np.ndarray:
    a = np.ascontiguousarray(seqs, dtype=np.int64)
    if a.ndim != 1:
        raise ValueError(f"{name} must be one-dimensional")
    return a


# ----------------------------------------------------------------------------
# device operations
# ----------------------------------------------------------------------------

def pa_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None):
    """k_new, v_new [T][H_kv][d]; slot_mapping int64 [T] (GPU tensors)."""
    torch = _torch()
    nb, H, bs, d = cache_geometry(k_cache, v_cache)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    T = slot_mapping.numel()
    if k_new.shape != (T, H, d) or v_new.shape != (T, H, d):
        raise ValueError("k_new / v_new shape mismatch")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("dtype mismatch")
    st = lib().pa_write_kv(_dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
                           _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                           _dev_ptr(slot_mapping, "slot_mapping"), T, nb, H, d, bs,
                           torch_dtype_code(k_cache), _stream_ptr(stream))
    _check(st, "pa_write_kv")


def pa_copy_blocks(k_cache, v_cache, pairs, stream=None):
    """pairs: int32 GPU tensor [P][2] of (src, dst)."""
    torch = _torch()
    nb, H, bs, d = cache_geometry(k_cache, v_cache)
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    if pairs.numel() % 2:
        raise ValueError("pairs must be [num_pairs][2]")
    P = pairs.numel() // 2
    if P == 0:
        return
    st = lib().pa_copy_blocks(_dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                              _dev_ptr(pairs, "pairs"), P, nb, H, d, bs,
                              torch_dtype_code(k_cache), _stream_ptr(stream))
    _check(st, "pa_copy_blocks")


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None):
    """Whole-block copies src -> dst between two caches of one geometry (GPU
    tensors or pinned CPU tensors); pairs int32 [P][2] (GPU or pinned)."""
    torch = _torch()
    nb_s, H, bs, d = cache_geometry(src_k, src_v)
    nb_d, H2, bs2, d2 = cache_geometry(dst_k, dst_v)
    if (H, bs, d) != (H2, bs2, d2) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination caches differ in geometry or dtype")
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    if pairs.numel() % 2:
        raise ValueError("pairs must be [num_pairs][2]")
    P = pairs.numel() // 2
    if P == 0:
        return
    st = lib().pa_swap_blocks(_any_ptr(src_k, "src_k"), _any_ptr(src_v, "src_v"), nb_s,
                              _any_ptr(dst_k, "dst_k"), _any_ptr(dst_v, "dst_v"), nb_d,
                              _any_ptr(pairs, "pairs"), P, H, d, bs, torch_dtype_code(src_k),
                              _stream_ptr(stream))
    _check(st, "pa_swap_blocks")


def pa_read_probe_partials() -> int:
    return int(lib().pa_read_probe_partials())


def pa_read_probe(buf, tile_bytes: int, tile_order, partials, nontemporal: bool = True,
                  stream=None):
    """Read-rate probe (measurement helper): reads buf (GPU uint8 tensor) as
    tiles of tile_bytes in tile_order (GPU int32 tensor); partials (GPU
    tensor of pa_read_probe_partials() x 16 bytes) receives each wave's XOR."""
    torch = _torch()
    if tile_order.dtype != torch.int32:
        raise TypeError("tile_order must be int32")
    num_tiles = buf.numel() * buf.element_size() // tile_bytes
    if partials.numel() * partials.element_size() < 16 * pa_read_probe_partials():
        raise ValueError("partials too small")
    st = lib().pa_read_probe(_dev_ptr(buf, "buf"), num_tiles, tile_bytes,
                             _dev_ptr(tile_order, "tile_order"), int(bool(nontemporal)),
                             _dev_ptr(partials, "partials"), _stream_ptr(stream))
    _check(st, "pa_read_probe")


def pa_decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int,
                             max_context_len: int, partition_size: int) -> int:
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                              max_context_len, partition_size))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
              scale: float, partition_size: int = 512, workspace=None, stream=None,
              flags: int = 0, seq_order=None):
    """out, q [B][H_q][d]; block_tables int32 [B][maxb]; context_lens int32 [B];
    seq_order: optional int32 GPU tensor [B] (issue order of the sequences)."""
    torch = _torch()
    nb, H_kv, bs, d, B, H_q = _check_decode_io(out, q, k_cache, v_cache)
    _check_tables(block_tables, context_lens, B)
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.numel() != B):
        raise ValueError("seq_order must be int32 [B]")
    need = pa_decode_workspace_size(B, H_q, d, max_context_len, partition_size)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if _nbytes(workspace) < need:
            raise ValueError("workspace too small")
        ws_ptr, ws_bytes = _dev_ptr(workspace, "workspace"), _nbytes(workspace)
    order_ptr = None if seq_order is None else _dev_ptr(seq_order, "seq_order")
    st = lib().pa_decode(_dev_ptr(out, "out"), _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"),
                         _dev_ptr(v_cache, "v_cache"), _dev_ptr(block_tables, "block_tables"),
                         block_tables.shape[1], _dev_ptr(context_lens, "context_lens"), order_ptr, B,
                         max_context_len, H_q, H_kv, d, bs, nb, float(scale), partition_size,
                         ws_ptr, ws_bytes, torch_dtype_code(q), flags, _stream_ptr(stream))
    _check(st, "pa_decode")
    return workspace


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens,
                      max_context_len: int, scale: float, partition_size: int = 512,
                      stream=None, flags: int = 0, seq_order=None):
    """pa_decode without a workspace argument: the partials go to the
    library's fixed per-GPU scratch (PA_NOALLOC_SCRATCH_BYTES); nothing is
    allocated.  Calls that overlap on one GPU race on that scratch."""
    torch = _torch()
    nb, H_kv, bs, d, B, H_q = _check_decode_io(out, q, k_cache, v_cache)
    _check_tables(block_tables, context_lens, B)
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.numel() != B):
        raise ValueError("seq_order must be int32 [B]")
    order_ptr = None if seq_order is None else _dev_ptr(seq_order, "seq_order")
    st = lib().pa_decode_noalloc(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                                 _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                 _dev_ptr(block_tables, "block_tables"), block_tables.shape[1],
                                 _dev_ptr(context_lens, "context_lens"), order_ptr, B,
                                 max_context_len, H_q, H_kv, d, bs, nb, float(scale),
                                 partition_size, torch_dtype_code(q), flags,
                                 _stream_ptr(stream))
    _check(st, "pa_decode_noalloc")


def pa_decode_order(block_tables: np.ndarray, context_lens: np.ndarray) -> np.ndarray:
    """Issue order for pa_decode from host tables int32 [B][maxb] and lengths
    int32 [B]: sharers of a first block together, longest work first."""
    tab = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = lens.size
    if tab.ndim != 2 or tab.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    out = np.empty(B, dtype=np.int32)
    _check(lib().pa_decode_order(_np_ptr(tab), tab.shape[1], _np_ptr(lens), B, _np_ptr(out)),
           "pa_decode_order")
    return out


def pa_cascade_plan(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                    num_q_heads: int, num_kv_heads: int, min_prefix: int = 512):
    """Host plan of the shared-prefix pass: (prefix_len int32 [B], groups int32
    [n][3], members int32 [m], max_prefix, max_members, max_rest)."""
    tab = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = lens.size
    if tab.ndim != 2 or tab.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    pre = np.zeros(max(1, B), dtype=np.int32)
    groups = np.zeros((max(1, B), 3), dtype=np.int32)
    members = np.zeros(max(1, B), dtype=np.int32)
    ng, mp, mm, mr = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().pa_cascade_plan(_np_ptr(tab), tab.shape[1], _np_ptr(lens), B, block_size,
                                 num_q_heads, num_kv_heads, min_prefix, _np_ptr(pre),
                                 _np_ptr(groups), _np_ptr(members), ctypes.byref(ng),
                                 ctypes.byref(mp), ctypes.byref(mm), ctypes.byref(mr)),
           "pa_cascade_plan")
    g = groups[:ng.value]
    nm = int(g[:, 1].sum()) if ng.value else 0
    return pre[:B], g, members[:nm], mp.value, mm.value, mr.value


def pa_decode_cascade_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int,
                                     max_context_len: int, partition_size: int) -> int:
    return int(lib().pa_decode_cascade_workspace_size(num_seqs, num_q_heads, head_dim,
                                                      max_context_len, partition_size))


def pa_decode_cascade(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                      scale: float, partition_size: int, prefix_len, groups, members,
                      max_prefix: int, max_members: int, max_rest: int, workspace, stream=None,
                      flags: int = 0, seq_order=None):
    """pa_decode with a shared-prefix plan (GPU int32 tensors from pa_cascade_plan)."""
    torch = _torch()
    nb, H_kv, bs, d, B, H_q = _check_decode_io(out, q, k_cache, v_cache)
    _check_tables(block_tables, context_lens, B)
    ng = groups.numel() // 3
    for t, name in ((prefix_len, "prefix_len"), (groups, "groups"), (members, "members")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if prefix_len.numel() != B:
        raise ValueError("prefix_len must have one entry per sequence")
    if seq_order is not None and (seq_order.dtype != torch.int32 or seq_order.numel() != B):
        raise ValueError("seq_order must be int32 [B]")
    st = lib().pa_decode_cascade(
        _dev_ptr(out, "out"), _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"),
        _dev_ptr(v_cache, "v_cache"), _dev_ptr(block_tables, "block_tables"),
        block_tables.shape[1], _dev_ptr(context_lens, "context_lens"),
        None if seq_order is None else _dev_ptr(seq_order, "seq_order"), B, max_context_len, H_q,
        H_kv, d, bs, nb, float(scale), partition_size, _dev_ptr(prefix_len, "prefix_len"),
        _dev_ptr(groups, "groups"), _dev_ptr(members, "members"), ng, max_prefix, max_members,
        max_rest, _dev_ptr(workspace, "workspace"), _nbytes(workspace), torch_dtype_code(q), flags,
        _stream_ptr(stream))
    _check(st, "pa_decode_cascade")


def pa_decode_step_staging_size(num_seqs: int, max_blocks_per_seq: int) -> int:
    return int(lib().pa_decode_step_staging_size(num_seqs, max_blocks_per_seq))


def _token_ids(tokens, n: int):
    """Optional token ids of the appended positions: None, or n ids (int32)."""
    if tokens is None:
        return None
    tk = np.ascontiguousarray(tokens, dtype=np.int32)
    if tk.ndim != 1 or tk.size != n:
        raise ValueError(f"tokens must be {n} ids, one per appended position")
    return tk


def pa_decode_step(pool: "Pool", seqs: np.ndarray, k_new, v_new, k_cache, v_cache, q, out,
                   scale: float, partition_size: int, max_blocks_per_seq: int, host_staging,
                   dev_staging, workspace, stream=None, tokens=None):
    """seqs: int64 numpy array; host_staging: pinned uint8 CPU tensor; dev_staging,
    workspace: uint8 GPU tensors; the rest GPU tensors as for pa_write_kv / pa_decode.
    tokens: optional token id of each sequence's new position (a prefix index
    attached to the pool then keeps indexing the blocks these sequences fill)."""
    nb, H_kv, bs, d, B, H_q = _check_decode_io(out, q, k_cache, v_cache)
    seqs = _seq_ids(seqs)
    if seqs.size != B:
        raise ValueError(f"{seqs.size} sequence ids for {B} query rows")
    tk = _token_ids(tokens, B)
    _check_new_kv(k_new, v_new, k_cache, B, H_kv, d)
    if not host_staging.is_pinned():
        raise ValueError("host_staging must be pinned host memory")
    sbytes = min(_nbytes(host_staging), _nbytes(dev_staging))
    st = lib().pa_decode_step(pool._h, _np_ptr(seqs), B, None if tk is None else _np_ptr(tk),
                              _dev_ptr(k_new, "k_new"),
                              _dev_ptr(v_new, "v_new"), _dev_ptr(k_cache, "k_cache"),
                              _dev_ptr(v_cache, "v_cache"), nb, H_kv, d, bs, _dev_ptr(q, "q"),
                              _dev_ptr(out, "out"), H_q, float(scale), partition_size,
                              max_blocks_per_seq, host_staging.data_ptr(),
                              _dev_ptr(dev_staging, "dev_staging"), sbytes,
                              _dev_ptr(workspace, "workspace"), _nbytes(workspace),
                              torch_dtype_code(q), _stream_ptr(stream))
    _check(st, "pa_decode_step")


def pa_beam_decode_step(pool: "Pool", old_beams, parents, new_beams, k_new, v_new, k_cache,
                        v_cache, q, out, scale: float, partition_size: int,
                        max_blocks_per_seq: int, host_staging, dev_staging, workspace,
                        stream=None, tokens=None):
    """One beam-search iteration in one native call (pool beam step, staging copy,
    copy-on-write, block write, decode).  Ids: int64 numpy arrays; k_new, v_new
    [len(new_beams)][H_kv][d], q / out [len(new_beams)][H_q][d] GPU tensors;
    tokens: optional token id of each new beam's new position."""
    nb, H_kv, bs, d, B, H_q = _check_decode_io(out, q, k_cache, v_cache)
    old = _seq_ids(old_beams, "old_beams")
    par = _seq_ids(parents, "parents")
    new = _seq_ids(new_beams, "new_beams")
    if par.size != new.size:
        raise ValueError("parents and new_beams differ in length")
    if new.size != B:
        raise ValueError(f"{new.size} new beams for {B} query rows")
    _check_new_kv(k_new, v_new, k_cache, B, H_kv, d)
    tk = _token_ids(tokens, B)
    if not host_staging.is_pinned():
        raise ValueError("host_staging must be pinned host memory")
    sbytes = min(_nbytes(host_staging), _nbytes(dev_staging))
    st = lib().pa_beam_decode_step(pool._h, _np_ptr(old), old.size, _np_ptr(par), _np_ptr(new),
                                   new.size, None if tk is None else _np_ptr(tk),
                                   _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
                                   _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                   nb, H_kv, d, bs, _dev_ptr(q, "q"), _dev_ptr(out, "out"), H_q,
                                   float(scale), partition_size, max_blocks_per_seq,
                                   host_staging.data_ptr(), _dev_ptr(dev_staging, "dev_staging"),
                                   sbytes, _dev_ptr(workspace, "workspace"), _nbytes(workspace),
                                   torch_dtype_code(q), _stream_ptr(stream))
    _check(st, "pa_beam_decode_step")


def sha256(data: bytes) -> bytes:
    out = (ctypes.c_uint8 * 32)()
    _check(lib().pa_sha256(data, len(data), out), "pa_sha256")
    return bytes(out)


def prefix_block_hash(parent, tokens, extra: bytes = b"") -> bytes:
    """Chain key of one block: parent (32 bytes or None), token ids, extra bytes."""
    tk = np.ascontiguousarray(tokens, dtype=np.int32)
    out = (ctypes.c_uint8 * 32)()
    par = None if parent is None else (ctypes.c_uint8 * 32).from_buffer_copy(parent)
    _check(lib().pa_prefix_block_hash(par, _np_ptr(tk), tk.size, extra or None, len(extra), out),
           "pa_prefix_block_hash")
    return bytes(out)


def pa_kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype: int) -> int:
    return int(lib().pa_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype))


# ----------------------------------------------------------------------------
# host block pool
# ----------------------------------------------------------------------------

def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Pool:
    """Owner of a pa_pool (host block pool)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.size != num_blocks:
                raise ValueError("free_order must have num_blocks entries")
        _check(lib().pa_pool_create(num_blocks, block_size, None if fo is None else _np_ptr(fo),
                                    ctypes.byref(h)), "pa_pool_create")
        self._h = h

    def close(self):
        if self._h:
            lib().pa_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self, seq: int) -> int:
        return lib().pa_seq_create(self._h, seq)

    def fork(self, parent: int, child: int) -> int:
        return lib().pa_seq_fork(self._h, parent, child)

    def free(self, seq: int) -> int:
        return lib().pa_seq_free(self._h, seq)

    def append(self, seq: int, k: int):
        """-> (status, slots int64[k], pairs int32[n][2])."""
        return self.append_batch(np.array([seq], dtype=np.int64), k)

    def append_batch(self, seqs, k: int, slots_out=None):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.size
        slots = slots_out if slots_out is not None else np.empty(max(1, n * k), dtype=np.int64)
        pairs = np.empty((max(1, n), 2), dtype=np.int32)
        npairs = ctypes.c_int(0)
        st = lib().pa_seq_append_batch(self._h, _np_ptr(seqs), n, k, _np_ptr(slots),
                                       _np_ptr(pairs), ctypes.byref(npairs))
        if st != PA_OK:
            return st, slots[:0], pairs[:0]
        return st, slots[:n * k], pairs[:npairs.value]

    def block_table(self, seq: int):
        nb, nt = ctypes.c_int(0), ctypes.c_int(0)
        st = lib().pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(nt))
        if st == PA_ERR_UNKNOWN_SEQ:
            raise KeyError(seq)
        out = np.empty(max(1, nb.value), dtype=np.int32)
        _check(lib().pa_seq_block_table(self._h, seq, _np_ptr(out), out.size, ctypes.byref(nb),
                                        ctypes.byref(nt)), "pa_seq_block_table")
        return out[:nb.value], nt.value

    def block_tables(self, seqs, maxb: int, out=None, lens_out=None):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.size
        out = out if out is not None else np.empty((n, maxb), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        _check(lib().pa_pool_block_tables(self._h, _np_ptr(seqs), n, _np_ptr(out), maxb,
                                          _np_ptr(lens)), "pa_pool_block_tables")
        return out, lens

    def refcount(self, block: int) -> int:
        return lib().pa_pool_refcount(self._h, block)

    def free_list(self):
        n = ctypes.c_int(0)
        out = np.empty(self.num_blocks, dtype=np.int32)
        _check(lib().pa_pool_free_list(self._h, _np_ptr(out), out.size, ctypes.byref(n)),
               "pa_pool_free_list")
        return out[:n.value]

    def stats(self):
        s = np.zeros(5, dtype=np.int64)
        _check(lib().pa_pool_stats(self._h, _np_ptr(s)), "pa_pool_stats")
        return dict(zip(("free", "used", "shared", "tokens", "copies"), s.tolist()))

    def beam_step(self, old_beams, parents, new_beams, tokens=None):
        """-> (status, slots int64 [n_new], pairs int32 [p][2])."""
        old = np.ascontiguousarray(old_beams, dtype=np.int64)
        par = np.ascontiguousarray(parents, dtype=np.int64)
        new = np.ascontiguousarray(new_beams, dtype=np.int64)
        tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(1, new.size), dtype=np.int64)
        pairs = np.empty((max(1, new.size), 2), dtype=np.int32)
        npairs = ctypes.c_int(0)
        st = lib().pa_seq_beam_step(self._h, _np_ptr(old), old.size, _np_ptr(par), _np_ptr(new),
                                    new.size, None if tk is None else _np_ptr(tk),
                                    _np_ptr(slots), _np_ptr(pairs), ctypes.byref(npairs))
        if st != PA_OK:
            return st, slots[:0], pairs[:0]
        return st, slots[:new.size], pairs[:npairs.value]

    # -- swapping ----------------------------------------------------------------
    def set_host_blocks(self, n: int) -> int:
        st = lib().pa_pool_set_host_blocks(self._h, n)
        if st == PA_OK:
            self.num_host_blocks = n
        return st

    def _swap(self, fn, seqs, cap=None):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        if cap is None:
            cap = 0
            for s in seqs.tolist():
                nb, nt = ctypes.c_int(0), ctypes.c_int(0)
                st = lib().pa_seq_block_table(self._h, s, None, 0, ctypes.byref(nb),
                                              ctypes.byref(nt))
                cap += nb.value if st in (PA_OK, PA_ERR_INVALID) else 0
        pairs = np.empty((max(1, cap), 2), dtype=np.int32)
        n = ctypes.c_int(0)
        st = fn(self._h, _np_ptr(seqs), seqs.size, _np_ptr(pairs), cap, ctypes.byref(n))
        return st, (pairs[:n.value] if st == PA_OK else pairs[:0])

    def swap_out(self, seqs, cap=None):
        """-> (status, pairs int32 [n][2] = {gpu block, host block})."""
        return self._swap(lib().pa_seq_swap_out, seqs, cap)

    def swap_in(self, seqs, cap=None):
        """-> (status, pairs int32 [n][2] = {host block, gpu block})."""
        return self._swap(lib().pa_seq_swap_in, seqs, cap)

    def is_swapped(self, seq: int) -> int:
        return lib().pa_seq_is_swapped(self._h, seq)

    # -- prefix reuse --------------------------------------------------------------
    def enable_prefix_cache(self, kind: int) -> int:
        return lib().pa_pool_enable_prefix_cache(self._h, kind)

    def create_cached(self, seq: int, tokens, salt: bytes = b"", extra: bytes = b""):
        """-> (status, cached_tokens, slots int64 [n - cached])."""
        tk = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(1, tk.size), dtype=np.int64)
        cached = ctypes.c_int(0)
        st = lib().pa_seq_create_cached(self._h, seq, _np_ptr(tk), tk.size, salt or None,
                                        len(salt), extra or None, len(extra),
                                        ctypes.byref(cached), _np_ptr(slots))
        if st != PA_OK:
            return st, 0, slots[:0]
        return st, cached.value, slots[:tk.size - cached.value]

    def append_tokens(self, seqs, tokens):
        """tokens [len(seqs)][k] -> (status, slots, pairs)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        tk = np.ascontiguousarray(tokens, dtype=np.int32).reshape(seqs.size, -1)
        n, k = seqs.size, tk.shape[1]
        slots = np.empty(max(1, n * k), dtype=np.int64)
        pairs = np.empty((max(1, n), 2), dtype=np.int32)
        npairs = ctypes.c_int(0)
        st = lib().pa_seq_append_tokens(self._h, _np_ptr(seqs), n, _np_ptr(tk), k, _np_ptr(slots),
                                        _np_ptr(pairs), ctypes.byref(npairs))
        if st != PA_OK:
            return st, slots[:0], pairs[:0]
        return st, slots[:n * k], pairs[:npairs.value]

    def prefix_stats(self):
        s = np.zeros(6, dtype=np.int64)
        _check(lib().pa_prefix_stats(self._h, _np_ptr(s)), "pa_prefix_stats")
        return dict(zip(("indexed", "evictable", "hits", "queried", "evicted", "nodes"),
                        s.tolist()))

    def host_stats(self):
        s = np.zeros(3, dtype=np.int64)
        _check(lib().pa_pool_host_stats(self._h, _np_ptr(s)), "pa_pool_host_stats")
        return dict(zip(("host_free", "host_used", "swapped"), s.tolist()))
