"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself:
  * a pure-Python scalar brute force (math.exp / math.fsum) on tiny inputs and
    on the tiny fp32 workload itself;
  * invariance of the output to a random permutation of the physical blocks
    (the pages: paging does not change the attention output);
  * equality with attention on the contiguous K/V the inputs were drawn as;
  * softmax weights summing to one; closed-form special cases;
  * the split-K log-sum-exp combine against the direct result;
  * the documented cache layout through hand-worked element offsets and a
    write/gather round trip.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle.pool_model import PoolModel
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers (test-side; they do not use the oracle's attention)
# ----------------------------------------------------------------------------

def brute_attention(q, K, V, scale):
    """Scalar attention. q: list[H_q][d]; K, V: list[n][H_kv][d] (python floats)."""
    H_q = len(q)
    n = len(K)
    H_kv = len(K[0]) if n else 1
    G = H_q // H_kv
    d = len(q[0])
    out = []
    for h in range(H_q):
        kv = h // G
        if n == 0:
            out.append([0.0] * d)
            continue
        z = [math.fsum(q[h][i] * K[t][kv][i] for i in range(d)) * scale for t in range(n)]
        m = max(z)
        w = [math.exp(zz - m) for zz in z]
        tot = math.fsum(w)
        out.append([math.fsum(w[t] * V[t][kv][i] for t in range(n)) / tot for i in range(d)])
    return out


def make_paged(seqs_kv, H, d, bs, dtype, num_blocks, rng):
    """Place each sequence's tokens through a PoolModel and the oracle's
    write_kv into a poisoned cache.  seqs_kv: list of (K, V) storage arrays
    [n][H][d].  Returns (kc, vc, tables, lens)."""
    st = synth.STORAGE[dtype]
    kc = np.zeros(A.k_cache_shape(num_blocks, H, bs, d, dtype), dtype=st)
    vc = np.zeros(A.v_cache_shape(num_blocks, H, bs, d, dtype), dtype=st)
    pois = synth.poison_bits(dtype)
    if dtype == "f32":
        kc.view(np.uint32)[...] = pois
        vc.view(np.uint32)[...] = pois
    else:
        kc.view(np.uint16)[...] = pois
        vc.view(np.uint16)[...] = pois
    pool = PoolModel(num_blocks, bs, rng.permutation(num_blocks))
    maxb = max(1, max(-(-len(k) // bs) for k, _ in seqs_kv))
    tables = np.full((len(seqs_kv), maxb), -1, dtype=np.int32)
    lens = np.zeros(len(seqs_kv), dtype=np.int32)
    for s, (k, v) in enumerate(seqs_kv):
        assert pool.create(s) == 0
        st_, slots, pairs = pool.append(s, len(k))
        assert st_ == 0 and not pairs
        A.write_kv(kc, vc, k, v, slots)
        t, n = pool.block_table(s)
        tables[s, :len(t)] = t
        lens[s] = n
    return kc, vc, tables, lens


def rand_seqs(rng, dtype, lens, H, d):
    out = []
    for n in lens:
        k = synth.cast_storage(rng.standard_normal((n, H, d), dtype=np.float32), dtype)
        v = synth.cast_storage(rng.standard_normal((n, H, d), dtype=np.float32), dtype)
        out.append((k, v))
    return out


# ----------------------------------------------------------------------------
# element decoding
# ----------------------------------------------------------------------------

def test_bf16_decoding_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    got = A.to_f64(bits, "bf16")
    assert got.tolist() == [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625]


def test_bf16_rounding_of_inputs_is_rne():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1.0 and 1.0078125: ties to even -> 1.0
    # 1 + 3*2^-8 lies between 1.0078125 and 1.015625: ties to even -> 1.015625
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = A.to_f64(synth.f32_to_bf16_bits(x), "bf16")
    assert got.tolist() == [1.0, 1.015625, 1.0078125]


# ----------------------------------------------------------------------------
# layout
# ----------------------------------------------------------------------------

def test_k_row_order():
    # tokens with bit 2 clear first, then with bit 2 set
    assert [A.k_row(t, 16) for t in range(16)] == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]
    order32 = sorted(range(32), key=lambda t: A.k_row(t, 32))
    assert order32 == [0, 1, 2, 3, 8, 9, 10, 11, 16, 17, 18, 19, 24, 25, 26, 27,
                       4, 5, 6, 7, 12, 13, 14, 15, 20, 21, 22, 23, 28, 29, 30, 31]


def test_layout_hand_worked_offsets():
    # bf16 (x = 8), H = 2, bs = 16, d = 16.  Tile = 16 * 16 = 256 elements.
    # K(b=1, h=1, t=3, i=10): tile (1*2+1)=3 -> 768; slab i//8 = 1 -> +1*16*8 = 128;
    #   token 3 sits in row 3 -> +3*8 = 24; lane i%8 = 2 -> 768+128+24+2 = 922
    assert A.k_offset(1, 1, 3, 10, H=2, bs=16, d=16, x=8) == 922
    # K(b=0, h=0, t=5, i=0): token 5 has bit 2 set -> row 8 + 0 + 1 = 9 -> 9*8 = 72
    assert A.k_offset(0, 0, 5, 0, H=2, bs=16, d=16, x=8) == 72
    # K(b=0, h=1, t=9, i=17) with d = 32: tile 256*2 = 512; slab 2 -> +2*128 = 256;
    #   token 9 (bit 2 clear) -> row 4 + 1 = 5 -> +40; lane 1 -> 809
    assert A.k_offset(0, 1, 9, 17, H=2, bs=16, d=32, x=8) == 809
    # V(b=1, h=1, t=11, i=5): tile 768; slab t//8 = 1 -> +1*16*8 = 128; dim 5 -> +40;
    #   t%8 = 3 -> 768+128+40+3 = 939
    assert A.v_offset(1, 1, 11, 5, H=2, bs=16, d=16, x=8) == 939
    # fp32 (x = 4), H = 1, bs = 16, d = 8:
    # K(0,0,t=5,i=6): slab 1 -> 64; token 5 -> row 9 -> 36; lane 2 -> 102
    assert A.k_offset(0, 0, 5, 6, H=1, bs=16, d=8, x=4) == 102
    # V(0,0,t=6,i=7): slab 1 -> 32; dim 7 -> 28; lane 2 -> 62
    assert A.v_offset(0, 0, 6, 7, H=1, bs=16, d=8, x=4) == 62


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_write_kv_places_elements_at_documented_offsets(dtype):
    rng = np.random.default_rng(5)
    H, bs, d, N = 2, 16, 16, 5
    x = A.vec_elems(dtype)
    st = synth.STORAGE[dtype]
    kc = np.zeros(A.k_cache_shape(N, H, bs, d, dtype), dtype=st)
    vc = np.zeros(A.v_cache_shape(N, H, bs, d, dtype), dtype=st)
    T = 20
    slots = rng.choice(N * bs, size=T, replace=False)
    kn = synth.cast_storage(rng.standard_normal((T, H, d), dtype=np.float32), dtype)
    vn = synth.cast_storage(rng.standard_normal((T, H, d), dtype=np.float32), dtype)
    A.write_kv(kc, vc, kn, vn, slots)
    kf, vf = kc.reshape(-1), vc.reshape(-1)
    for j, s in enumerate(slots):
        b, t = divmod(int(s), bs)
        for h in range(H):
            for i in range(d):
                assert kf[A.k_offset(b, h, t, i, H, bs, d, x)] == kn[j, h, i]
                assert vf[A.v_offset(b, h, t, i, H, bs, d, x)] == vn[j, h, i]


@pytest.mark.parametrize("dtype,bs", [("f32", 16), ("bf16", 16), ("f16", 32)])
def test_write_then_gather_round_trip(dtype, bs):
    rng = np.random.default_rng(7)
    H, d = 3, 64
    lens = [1, bs, bs + 1, 3 * bs - 1, 50]
    seqs = rand_seqs(rng, dtype, lens, H, d)
    kc, vc, tables, L = make_paged(seqs, H, d, bs, dtype, 40, rng)
    for s, (k, v) in enumerate(seqs):
        K, V = A.gather_sequence(kc, vc, tables[s], int(L[s]), dtype)
        assert np.array_equal(K, A.to_f64(k, dtype))
        assert np.array_equal(V, A.to_f64(v, dtype))


def test_write_kv_skips_negative_slots():
    rng = np.random.default_rng(8)
    H, bs, d = 1, 16, 8
    kc = np.zeros(A.k_cache_shape(2, H, bs, d, "f32"), dtype=np.float32)
    vc = np.zeros(A.v_cache_shape(2, H, bs, d, "f32"), dtype=np.float32)
    kn = rng.standard_normal((3, H, d)).astype(np.float32)
    A.write_kv(kc, vc, kn, kn, [-1, 5, -7])
    K, _ = A.gather_sequence(kc, vc, [0], 6, "f32")
    assert np.array_equal(K[5], kn[1].astype(np.float64))
    assert np.count_nonzero(kc) == H * d


def test_copy_blocks_copies_whole_blocks_in_order():
    rng = np.random.default_rng(9)
    H, bs, d, N = 2, 16, 16, 6
    kc = synth.cast_storage(rng.standard_normal(A.k_cache_shape(N, H, bs, d, "bf16")).astype(np.float32), "bf16")
    vc = synth.cast_storage(rng.standard_normal(A.v_cache_shape(N, H, bs, d, "bf16")).astype(np.float32), "bf16")
    k0, v0 = kc.copy(), vc.copy()
    A.copy_blocks(kc, vc, [(1, 4), (2, 5)])
    assert np.array_equal(kc[4], k0[1]) and np.array_equal(vc[4], v0[1])
    assert np.array_equal(kc[5], k0[2]) and np.array_equal(vc[5], v0[2])
    for b in (0, 1, 2, 3):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])


def _token_values(N, H, bs, d, tag):
    """A value for every (block, head, token, dim) that names it: distinct
    across positions and across K / V (tag), exact in fp32."""
    b, h, t, i = np.meshgrid(np.arange(N), np.arange(H), np.arange(bs), np.arange(d),
                             indexing="ij")
    return (tag * 1e6 + b * 1e4 + h * 1e3 + t * 10 + i * 0.0625).astype(np.float32)


@pytest.mark.parametrize("bs", [16, 32])
def test_swap_blocks_moves_whole_k_and_v_blocks_from_source_to_destination(bs):
    """Swap to host memory and back (tonho.wtf, "a ideia": the cache can be
    swapped to CPU RAM; "como funciona": a preempted sequence comes back by
    swapping in, all of its blocks).  Every element is checked through the
    hand-pinned per-element offsets, not through block slicing: a reversed
    pair direction, a K-only copy, a partial block or a write outside the
    listed destinations each fail here."""
    H, d, Ng, Nh = 2, 8, 7, 5
    x = A.vec_elems("f32")
    kval = _token_values(Ng, H, bs, d, 1)
    vval = _token_values(Ng, H, bs, d, 2)
    gk = np.zeros(A.k_cache_shape(Ng, H, bs, d, "f32"), np.float32)
    gv = np.zeros(A.v_cache_shape(Ng, H, bs, d, "f32"), np.float32)
    # fill the device-side cache element by element at the documented offsets
    gkf, gvf = gk.reshape(-1), gv.reshape(-1)
    for b in range(Ng):
        for h in range(H):
            for t in range(bs):
                for i in range(d):
                    gkf[A.k_offset(b, h, t, i, H, bs, d, x)] = kval[b, h, t, i]
                    gvf[A.v_offset(b, h, t, i, H, bs, d, x)] = vval[b, h, t, i]
    poison = np.float32(-7.5)
    hk = np.full(A.k_cache_shape(Nh, H, bs, d, "f32"), poison, np.float32)
    hv = np.full(A.v_cache_shape(Nh, H, bs, d, "f32"), poison, np.float32)
    g0k, g0v = gk.copy(), gv.copy()

    out_pairs = [(6, 0), (2, 3), (4, 1)]          # device block -> host block
    A.swap_blocks(gk, gv, hk, hv, out_pairs)
    # the source cache is only read
    assert np.array_equal(gk, g0k) and np.array_equal(gv, g0v)
    hkf, hvf = hk.reshape(-1), hv.reshape(-1)
    for src, dst in out_pairs:
        for h in range(H):
            for t in range(bs):
                for i in range(d):
                    assert hkf[A.k_offset(dst, h, t, i, H, bs, d, x)] == kval[src, h, t, i]
                    assert hvf[A.v_offset(dst, h, t, i, H, bs, d, x)] == vval[src, h, t, i]
    # host blocks not listed as a destination keep their contents
    for b in (2, 4):
        assert np.all(hk[b] == poison) and np.all(hv[b] == poison)

    # back in, into other device blocks: the round trip restores each block
    in_pairs = [(0, 5), (3, 0), (1, 1)]            # host block -> device block
    A.swap_blocks(hk, hv, gk, gv, in_pairs)
    for (gsrc, _), (_, gdst) in zip(out_pairs, in_pairs):
        assert np.array_equal(gk[gdst], g0k[gsrc]) and np.array_equal(gv[gdst], g0v[gsrc])
    for b in (2, 3, 4, 6):
        assert np.array_equal(gk[b], g0k[b]) and np.array_equal(gv[b], g0v[b])


def test_swap_blocks_applies_pairs_in_order():
    """Pairs are applied one after the other: a destination named twice ends
    with the second source; one source may feed several destinations."""
    H, bs, d = 1, 16, 8
    src_k = _token_values(3, H, bs, d, 1)
    src_v = _token_values(3, H, bs, d, 2)
    sk = np.ascontiguousarray(src_k.reshape(A.k_cache_shape(3, H, bs, d, "f32")))
    sv = np.ascontiguousarray(src_v.reshape(A.v_cache_shape(3, H, bs, d, "f32")))
    dk = np.zeros(A.k_cache_shape(4, H, bs, d, "f32"), np.float32)
    dv = np.zeros(A.v_cache_shape(4, H, bs, d, "f32"), np.float32)
    A.swap_blocks(sk, sv, dk, dv, [(0, 2), (1, 2), (1, 3)])
    assert np.array_equal(dk[2], sk[1]) and np.array_equal(dv[2], sv[1])
    assert np.array_equal(dk[3], sk[1]) and np.array_equal(dv[3], sv[1])
    assert not np.any(dk[:2]) and not np.any(dv[:2])


# ----------------------------------------------------------------------------
# attention: brute force
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("H_q,H_kv", [(1, 1), (2, 1), (4, 2), (6, 2)])
def test_oracle_matches_scalar_brute_force(H_q, H_kv):
    rng = np.random.default_rng(11 + H_q)
    d, bs = 8, 4
    lens = [1, 3, 4, 17, 40]
    seqs = rand_seqs(rng, "f32", lens, H_kv, d)
    kc, vc, tables, L = make_paged(seqs, H_kv, d, bs, "f32", 40, rng)
    q = rng.standard_normal((len(lens), H_q, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    got = A.paged_decode(q, kc, vc, tables, L, scale, "f32")
    for s, (k, v) in enumerate(seqs):
        ref = brute_attention(q[s].astype(float).tolist(), k.astype(float).tolist(),
                              v.astype(float).tolist(), scale)
        assert np.max(np.abs(got[s] - np.array(ref))) <= 1e-12


def test_tiny_fp32_workload_matches_brute_force():
    wl = synth.WORKLOADS["tiny_mha_fp32"]
    sc = synth.build_scenario(wl)
    rng = np.random.default_rng(0)
    seqs = []
    for op in sc.ops:
        if op[0] == "append":
            seqs.append(sc.values(op[1]))
    kc, vc, tables, L = make_paged(seqs, wl.h_kv, wl.head_dim, wl.block_size, wl.dtype,
                                   wl.pool_blocks, rng)
    got = A.paged_decode(sc.q, kc, vc, tables, L, wl.scale, wl.dtype)
    for s, (k, v) in enumerate(seqs):
        ref = brute_attention(sc.q[s].astype(float).tolist(), k.astype(float).tolist(),
                              v.astype(float).tolist(), wl.scale)
        assert np.max(np.abs(got[s] - np.array(ref))) <= 1e-12


# ----------------------------------------------------------------------------
# invariances and special cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_permutation_of_physical_blocks_leaves_output_bit_identical(dtype):
    rng = np.random.default_rng(21)
    H_q, H_kv, d, bs, N = 8, 2, 64, 16, 48
    lens = [5, 16, 33, 100, 250]
    seqs = rand_seqs(rng, dtype, lens, H_kv, d)
    kc, vc, tables, L = make_paged(seqs, H_kv, d, bs, dtype, N, rng)
    q = synth.cast_storage(rng.standard_normal((len(lens), H_q, d), dtype=np.float32), dtype)
    out1 = A.paged_decode(q, kc, vc, tables, L, 0.125, dtype)
    perm = rng.permutation(N)                 # block b moves to perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = A.paged_decode(q, kc2, vc2, t2, L, 0.125, dtype)
    assert np.array_equal(out1, out2)


def test_equals_attention_on_contiguous_inputs():
    rng = np.random.default_rng(22)
    H_q, H_kv, d, bs = 4, 4, 64, 16
    lens = [7, 64, 129]
    seqs = rand_seqs(rng, "bf16", lens, H_kv, d)
    kc, vc, tables, L = make_paged(seqs, H_kv, d, bs, "bf16", 30, rng)
    q = synth.cast_storage(rng.standard_normal((3, H_q, d), dtype=np.float32), "bf16")
    out = A.paged_decode(q, kc, vc, tables, L, 0.125, "bf16")
    for s, (k, v) in enumerate(seqs):
        direct = A.attention_contiguous(A.to_f64(q[s], "bf16"), A.to_f64(k, "bf16"),
                                        A.to_f64(v, "bf16"), 0.125)
        assert np.array_equal(out[s], direct)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(23)
    K = rng.standard_normal((300, 2, 32))
    V = rng.standard_normal((300, 2, 32))
    q = rng.standard_normal((4, 32)) * 3
    _, P = A.attention_contiguous(q, K, V, 1 / math.sqrt(32), return_p=True)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(axis=1) - 1)) <= 1e-12


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(24)
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    q = rng.standard_normal((4, 16))
    out = A.attention_contiguous(q, K, V, 0.25)
    for h in range(4):
        assert np.array_equal(out[h], V[0, h // 2])


def test_zero_query_or_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(25)
    V = rng.standard_normal((37, 1, 16))
    K = rng.standard_normal((37, 1, 16))
    out = A.attention_contiguous(np.zeros((1, 16)), K, V, 0.25)
    assert np.max(np.abs(out[0] - V[:, 0].mean(axis=0))) <= 1e-12
    Keq = np.repeat(K[:1], 37, axis=0)
    out = A.attention_contiguous(rng.standard_normal((1, 16)), Keq, V, 0.25)
    assert np.max(np.abs(out[0] - V[:, 0].mean(axis=0))) <= 1e-12


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(26)
    K = rng.standard_normal((50, 1, 16)) * 0.01
    V = rng.standard_normal((50, 1, 16))
    q = np.zeros((1, 16))
    q[0, 3] = 1e4
    K[17, 0, 3] = 1.0
    out = A.attention_contiguous(q, K, V, 1.0)
    assert np.max(np.abs(out[0] - V[17, 0])) <= 1e-12


def test_grouped_heads_equal_mha_with_duplicated_kv_heads():
    rng = np.random.default_rng(27)
    H_q, H_kv, d, n = 8, 2, 16, 45
    G = H_q // H_kv
    K = rng.standard_normal((n, H_kv, d))
    V = rng.standard_normal((n, H_kv, d))
    q = rng.standard_normal((H_q, d))
    gqa = A.attention_contiguous(q, K, V, 0.25)
    Kd = np.stack([K[:, h // G] for h in range(H_q)], axis=1)
    Vd = np.stack([V[:, h // G] for h in range(H_q)], axis=1)
    mha = A.attention_contiguous(q, Kd, Vd, 0.25)
    assert np.array_equal(gqa, mha)
    # and the grouping is contiguous: head 1 reads KV head 0, not KV head 1
    assert not np.allclose(gqa[1], A.attention_contiguous(q[1:2], K[:, 1:2], V[:, 1:2], 0.25)[0])


def test_zero_context_gives_zero_row():
    q = np.ones((2, 8))
    out = A.attention_contiguous(q, np.zeros((0, 1, 8)), np.zeros((0, 1, 8)), 0.3)
    assert np.array_equal(out, np.zeros((2, 8)))


@pytest.mark.parametrize("P", [1, 7, 32, 512])
def test_split_k_combine_equals_direct(P):
    rng = np.random.default_rng(28)
    n = 1000
    K = rng.standard_normal((n, 2, 32))
    V = rng.standard_normal((n, 2, 32))
    q = rng.standard_normal((4, 32)) * 2
    direct = A.attention_contiguous(q, K, V, 0.2)
    split = A.split_attention(q, K, V, 0.2, P)
    assert np.max(np.abs(direct - split)) <= 1e-12


def test_poisoned_tail_and_padding_are_never_read():
    rng = np.random.default_rng(29)
    H, d, bs = 2, 16, 16
    seqs = rand_seqs(rng, "bf16", [5, 20], H, d)
    kc, vc, tables, L = make_paged(seqs, H, d, bs, "bf16", 8, rng)
    q = synth.cast_storage(rng.standard_normal((2, H, d), dtype=np.float32), "bf16")
    out = A.paged_decode(q, kc, vc, tables, L, 0.25, "bf16")
    assert np.all(np.isfinite(out))          # the NaN poison in unfilled slots is not read
    t2 = np.concatenate([tables, np.full((2, 3), 12345, dtype=np.int32)], axis=1)
    out2 = A.paged_decode(q, kc, vc, t2, L, 0.25, "bf16")
    assert np.array_equal(out, out2)         # entries past ceil(ctx/bs) are not read
