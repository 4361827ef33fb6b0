"""The usage example of README.md, run as a test: a manager with two
sequences that share a prompt, one decode iteration through the manager and
one through the one-call step, each checked against attention computed in
float32 from the K/V the example appended."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def reference(q, k, v, scale):
    """softmax(q K^T scale) V per query head, GQA groups of contiguous heads."""
    import torch
    q, k, v = q.float().cpu(), k.float().cpu(), v.float().cpu()     # [H_q][d], [n][H_kv][d]
    G = q.shape[0] // k.shape[1]
    kk = k.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()   # [H_q][n][d]
    vv = v.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    p = torch.softmax(torch.einsum("hd,hnd->hn", q, kk) * scale, dim=-1)
    return torch.einsum("hn,hnd->hd", p, vv)


def test_readme_example():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # --- the example ---------------------------------------------------------
    import paged_kv_cache_12_amd as pa
    from paged_kv_cache_12_amd.manager import PagedKVCache

    H_q, H_kv, d, bs = 32, 8, 128, 16
    bf16 = dict(device="cuda", dtype=torch.bfloat16)
    cache = PagedKVCache(num_blocks=256, block_size=bs, num_kv_heads=H_kv, head_dim=d,
                         dtype="bf16")
    cache.create(0)
    k = torch.randn(100, H_kv, d, **bf16)               # a 100-token prompt
    v = torch.randn(100, H_kv, d, **bf16)
    cache.append([0], 100, k, v)                         # slots, block write
    cache.fork(0, 1)                                     # sequence 1 shares its blocks

    # one decode iteration through the manager: append one token to each
    # (copy-on-write of the shared, partly filled last block), then attend
    kn, vn = torch.randn(2, H_kv, d, **bf16), torch.randn(2, H_kv, d, **bf16)
    slots, pairs = cache.append([0, 1], 1, kn, vn)
    q = torch.randn(2, H_q, d, **bf16)
    out, tables, lens = cache.decode(q, [0, 1], scale=d ** -0.5)

    # the next iteration in one native call (pool step, metadata copy,
    # copy-on-write, decode with the block write folded in)
    seqs = np.array([0, 1], dtype=np.int64)
    maxb = 64
    nbytes = pa.pa_decode_step_staging_size(len(seqs), maxb)
    host_staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev_staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    workspace = torch.empty(max(256, pa.pa_decode_workspace_size(2, H_q, d, maxb * bs, 512)),
                            dtype=torch.uint8, device="cuda")
    kn2, vn2 = torch.randn(2, H_kv, d, **bf16), torch.randn(2, H_kv, d, **bf16)
    q2 = torch.randn(2, H_q, d, **bf16)
    out2 = torch.empty_like(q2)
    pa.pa_decode_step(cache.pool, seqs, kn2, vn2, cache.k_cache, cache.v_cache, q2, out2,
                      d ** -0.5, 512, maxb, host_staging, dev_staging, workspace)
    torch.cuda.synchronize()
    # --- checks ----------------------------------------------------------------
    assert len(pairs) == 1 and list(lens) == [101, 101]
    for i in range(2):
        ks = torch.cat([k, kn[i:i + 1]])
        vs = torch.cat([v, vn[i:i + 1]])
        ref = reference(q[i], ks, vs, d ** -0.5)
        assert (out[i].float().cpu() - ref).abs().max().item() < 2e-2
        ks2 = torch.cat([ks, kn2[i:i + 1]])
        vs2 = torch.cat([vs, vn2[i:i + 1]])
        ref2 = reference(q2[i], ks2, vs2, d ** -0.5)
        assert (out2[i].float().cpu() - ref2).abs().max().item() < 2e-2
