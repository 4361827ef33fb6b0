"""The Python binding's argument checks (CPU only): a q, out, k_new or v_new
whose dtype differs from the cache's, a shape that does not match the cache
geometry, or a sequence-id array that does not match the query rows is
refused with TypeError / ValueError before any pointer reaches libpa.so."""
import numpy as np
import pytest
import torch

import paged_kv_cache_12_amd as pa

H_KV, BS, D, NB = 2, 16, 64, 8


def cache(dtype=torch.bfloat16):
    x = 16 // torch.empty((), dtype=dtype).element_size()
    k = torch.zeros((NB, H_KV, D // x, BS, x), dtype=dtype)
    v = torch.zeros((NB, H_KV, BS // x, D, x), dtype=dtype)
    return k, v


def decode_args(B=3, H_q=4, dtype=torch.bfloat16, q_dtype=None, out_dtype=None,
                out_shape=None):
    k, v = cache(dtype)
    q = torch.zeros((B, H_q, D), dtype=q_dtype or dtype)
    out = torch.zeros(out_shape or (B, H_q, D), dtype=out_dtype or dtype)
    tab = torch.zeros((B, 2), dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    return out, q, k, v, tab, lens


@pytest.mark.parametrize("which", ["q", "out"])
@pytest.mark.parametrize("cache_dtype,other", [(torch.bfloat16, torch.float32),
                                               (torch.float16, torch.bfloat16),
                                               (torch.float32, torch.float16)])
def test_decode_refuses_dtype_mismatch(which, cache_dtype, other):
    kw = {"q_dtype": other} if which == "q" else {"out_dtype": other}
    out, q, k, v, tab, lens = decode_args(dtype=cache_dtype, **kw)
    with pytest.raises(TypeError):
        pa.pa_decode(out, q, k, v, tab, lens, 16, 0.125, 0)
    with pytest.raises(TypeError):
        pa.pa_decode_cascade(out, q, k, v, tab, lens, 16, 0.125, 0, lens, lens, lens, 0, 1, 0,
                             torch.zeros(256, dtype=torch.uint8))


@pytest.mark.parametrize("out_shape", [(3, 4, 32), (2, 4, 64), (3, 8, 64)])
def test_decode_refuses_out_shape_mismatch(out_shape):
    out, q, k, v, tab, lens = decode_args(out_shape=out_shape)
    with pytest.raises(ValueError):
        pa.pa_decode(out, q, k, v, tab, lens, 16, 0.125, 0)


def test_decode_refuses_wrong_head_dim_and_group():
    out, q, k, v, tab, lens = decode_args()
    bad = torch.zeros((3, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.pa_decode(bad, bad, k, v, tab, lens, 16, 0.125, 0)
    odd = torch.zeros((3, 3, D), dtype=torch.bfloat16)    # 3 query heads over 2 KV heads
    with pytest.raises(ValueError):
        pa.pa_decode(odd, odd, k, v, tab, lens, 16, 0.125, 0)


def test_decode_refuses_table_mismatch():
    out, q, k, v, tab, lens = decode_args()
    with pytest.raises(TypeError):
        pa.pa_decode(out, q, k, v, tab.to(torch.int64), lens, 16, 0.125, 0)
    with pytest.raises(ValueError):
        pa.pa_decode(out, q, k, v, tab[:2], lens, 16, 0.125, 0)
    with pytest.raises(ValueError):
        pa.pa_decode(out, q, k, v, tab, lens, 16, 0.125, 0,
                     seq_order=torch.zeros(2, dtype=torch.int32))


def test_decode_with_matching_cpu_arguments_still_needs_gpu_memory():
    """All checks pass: the next refusal is the pointer check (GPU memory)."""
    out, q, k, v, tab, lens = decode_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        pa.pa_decode(out, q, k, v, tab, lens, 16, 0.125, 0)


def step_args(B=3, H_q=4, dtype=torch.bfloat16, new_dtype=None, new_rows=None):
    out, q, k, v, _, _ = decode_args(B, H_q, dtype)
    n = B if new_rows is None else new_rows
    kn = torch.zeros((n, H_KV, D), dtype=new_dtype or dtype)
    vn = torch.zeros((n, H_KV, D), dtype=new_dtype or dtype)
    return out, q, k, v, kn, vn


def call_step(seqs, out, q, k, v, kn, vn):
    pool = pa.Pool(NB, BS)
    stage = torch.zeros(64, dtype=torch.uint8)
    pa.pa_decode_step(pool, seqs, kn, vn, k, v, q, out, 0.125, 0, 2, stage, stage, stage)


@pytest.mark.parametrize("kw", [dict(new_dtype=torch.float32), dict(new_dtype=torch.float16),
                                dict(new_rows=2)])
def test_decode_step_refuses_new_kv_mismatch(kw):
    out, q, k, v, kn, vn = step_args(**kw)
    with pytest.raises(TypeError if "new_dtype" in kw else ValueError):
        call_step(np.arange(3), out, q, k, v, kn, vn)


def test_decode_step_refuses_short_or_2d_seq_ids():
    out, q, k, v, kn, vn = step_args()
    with pytest.raises(ValueError):
        call_step(np.arange(2), out, q, k, v, kn, vn)
    with pytest.raises(ValueError):
        call_step(np.arange(6).reshape(3, 2), out, q, k, v, kn, vn)


def test_decode_step_converts_seq_ids_to_int64():
    """int32 ids are converted (not read as int64 past their end): every
    check passes and the call reaches the pinned-memory check."""
    out, q, k, v, kn, vn = step_args()
    with pytest.raises(ValueError, match="pinned"):
        call_step(np.arange(3, dtype=np.int32), out, q, k, v, kn, vn)


def test_steps_refuse_token_ids_of_the_wrong_count():
    """Token ids: one per appended position, checked before the pool or any
    pointer is touched."""
    out, q, k, v, kn, vn = step_args()
    pool = pa.Pool(NB, BS)
    stage = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="tokens"):
        pa.pa_decode_step(pool, np.arange(3), kn, vn, k, v, q, out, 0.125, 0, 2, stage, stage,
                          stage, tokens=[1, 2])
    with pytest.raises(ValueError, match="tokens"):
        pa.pa_decode_step(pool, np.arange(3), kn, vn, k, v, q, out, 0.125, 0, 2, stage, stage,
                          stage, tokens=[[1], [2], [3]])
    with pytest.raises(ValueError, match="tokens"):
        pa.pa_beam_decode_step(pool, [0], [0, 0, 0], [1, 2, 3], kn, vn, k, v, q, out, 0.125, 0,
                               2, stage, stage, stage, tokens=[5])
    # the right count passes every check and reaches the pinned-memory one
    with pytest.raises(ValueError, match="pinned"):
        pa.pa_decode_step(pool, np.arange(3), kn, vn, k, v, q, out, 0.125, 0, 2, stage, stage,
                          stage, tokens=[1, 2, 3])


def test_beam_step_refuses_mismatches():
    out, q, k, v, kn, vn = step_args(B=4)
    pool = pa.Pool(NB, BS)
    stage = torch.zeros(64, dtype=torch.uint8)
    args = (k, v, q, out, 0.125, 0, 2, stage, stage, stage)
    with pytest.raises(ValueError):     # 3 new beams for 4 query rows
        pa.pa_beam_decode_step(pool, [0], [0, 0, 0], [1, 2, 3], kn, vn, *args)
    with pytest.raises(ValueError):     # parents and new beams differ in length
        pa.pa_beam_decode_step(pool, [0], [0, 0], [1, 2, 3, 4], kn, vn, *args)
    with pytest.raises(TypeError):
        pa.pa_beam_decode_step(pool, [0], [0] * 4, [1, 2, 3, 4], kn.float(), vn, *args)


def test_write_and_copy_refuse_mismatches():
    k, v = cache()
    with pytest.raises(TypeError):
        pa.pa_write_kv(torch.zeros((2, H_KV, D)), torch.zeros((2, H_KV, D)), k, v,
                       torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError):
        pa.pa_copy_blocks(k, v, torch.zeros(3, dtype=torch.int32))
