"""GPU check of the read-rate probe (pa_read_probe): the XOR of its per-wave
partials equals the XOR of exactly the tiles its order names, so the rate
bench.py reports is the rate of reading every tile once."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    import paged_kv_cache_12_amd as pa
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


def _xor_rows(a):
    return np.bitwise_xor.reduce(a.reshape(-1, 4), axis=0)


@pytest.mark.parametrize("nontemporal", [True, False])
def test_read_probe_reads_each_listed_tile_once(nontemporal):
    import torch
    import paged_kv_cache_12_amd as pa
    tile = 4096
    host = np.random.default_rng(5).integers(0, 2 ** 32, (16 << 20) // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    n = host.nbytes // tile
    partials = torch.empty(16 * pa.pa_read_probe_partials(), dtype=torch.uint8, device="cuda")
    tiles = host.reshape(n, tile // 4)
    # a permutation: every tile once
    order = np.random.default_rng(6).permutation(n).astype(np.int32)
    pa.pa_read_probe(buf, tile, torch.from_numpy(order).cuda(), partials, nontemporal)
    torch.cuda.synchronize()
    got = _xor_rows(partials.cpu().numpy().view(np.uint32))
    assert np.array_equal(got, _xor_rows(tiles))
    # repeated and out-of-range entries: tiles 0, 0 and 5 (the rest skipped)
    order = np.full(n, -1, dtype=np.int32)
    order[:4] = [0, 0, 5, n + 3]
    pa.pa_read_probe(buf, tile, torch.from_numpy(order).cuda(), partials, nontemporal)
    torch.cuda.synchronize()
    got = _xor_rows(partials.cpu().numpy().view(np.uint32))
    assert np.array_equal(got, _xor_rows(tiles[5]))
