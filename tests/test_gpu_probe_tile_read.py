"""The tile-read measurement probe on the GPU: every built (tile bytes, paths, team) variant
launches over a small pool, reads what it reports, and leaves the sink word alone on data
that cannot fold to its trigger value (all-zero pools fold to zero).  Block ids outside the
pool read block 0 instead."""
import numpy as np
import pytest

import paged_kv_decode_blocks_amd as pkv

pytestmark = pytest.mark.gpu

BUILT = ([(1024, p, 4) for p in (0, 1, 4, 5, 6, 7)] + [(2048, p, 4) for p in (0, 1, 5, 7)] +
         [(4096, p, 4) for p in (0, 1, 5)] + [(1024, p, d) for p in (0, 4, 6, 7) for d in (2, 8)])


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("team", [1, 2, 4])
@pytest.mark.parametrize("tile,paths,depth", BUILT)
def test_every_variant_reads_and_leaves_the_sink(torch_dev, tile, paths, depth, team):
    torch = torch_dev
    heads, n_blocks = 8, 40
    kp = torch.zeros(n_blocks * heads * tile // 4, dtype=torch.int32, device="cuda")
    vp = torch.zeros_like(kp)
    ks = torch.zeros(n_blocks * heads * 64 // 4, dtype=torch.int32, device="cuda")
    vs = torch.zeros_like(ks)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ids = np.random.default_rng(tile + paths + team + depth).integers(0, n_blocks, size=203).astype(np.int32)
    ids[[5, 77, 150]] = (-1, n_blocks, 1 << 30)      # outside the pool: read block 0
    ids_t = torch.from_numpy(ids).cuda()
    scales = bool(paths & 4) or tile == 1024
    for grid in (1, 3, 64):
        n = pkv.probe_tile_read(kp, vp, ids_t, sink, heads=heads, tile_bytes=tile, team=team, paths=paths,
                                depth=depth, k_scale=ks if scales else None, v_scale=vs if scales else None,
                                grid=grid)
        assert n == 203 * team * (2 * tile + (128 if scales else 0))
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_unbuilt_variant_and_bad_team_raise(torch_dev):
    torch = torch_dev
    kp = torch.zeros(8 * 6 * 4096 // 4, dtype=torch.int32, device="cuda")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError):
        pkv.probe_tile_read(kp, kp, ids, sink, heads=8, tile_bytes=4096, paths=7, k_scale=kp, v_scale=kp)
    with pytest.raises(pkv.PkvError):
        pkv.probe_tile_read(kp, kp, ids, sink, heads=6, tile_bytes=1024, team=4)
    assert pkv.probe_tile_read(kp, kp, ids, sink, heads=6, tile_bytes=1024, team=2, n_items=0) == 0
