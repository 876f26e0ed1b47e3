"""GPU index builder (K0) against the oracle's tables: bit-exact, every packing, every workload geometry."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import DEV, say

pytestmark = pytest.mark.gpu


def _compare(coords, block, r):
    ix = p3.build_index(coords.to(DEV), block, r)
    tab = ix.tables()
    ref = oracle.build_index(coords.numpy(), block, r)
    for v, rv in enumerate(ref):
        assert np.array_equal(tab["token_block"][v].cpu().numpy(), rv["token_block"])
        assert np.array_equal(tab["canon"][v].cpu().numpy(), rv["canon"])
        assert np.array_equal(tab["perm"][v].cpu().numpy(), rv["perm"])
        assert np.array_equal(tab["nbr"][v].cpu().numpy(), rv["nbr"])
        origin, extent = ix.geometry(v)
        assert origin == tuple(rv["origin"]) and extent == tuple(rv["extent"])
    return ix


@pytest.mark.parametrize("name", ["tiny", "16k", "65k", "524k"])
def test_tables_bit_exact_on_workload_geometries(name):
    w = si.WORKLOADS[name]
    say(f"index {name}")
    perms = [si.packing_permutation(w.grid, w.packing, block=w.block, seed=w.seed, volume=v) for v in range(w.batch)]
    rc = si.raster_coords(w.grid)
    coords = torch.from_numpy(np.stack([rc[p] for p in perms]))
    _compare(coords, w.block, w.radius)


@pytest.mark.parametrize("packing", si.PACKINGS)
@pytest.mark.parametrize("grid,block,r", [((8, 12, 16), (2, 2, 4), 1), ((4, 8, 8), (4, 4, 4), 2),
                                          ((6, 8, 10), (2, 4, 2), 0), ((16, 8, 8), (4, 4, 4), 3)])
def test_tables_bit_exact_every_packing(packing, grid, block, r):
    perm = si.packing_permutation(grid, packing, block=block, seed=5)
    coords = torch.from_numpy((si.raster_coords(grid)[perm] + np.array([-3, 11, 40], dtype=np.int32))[None])
    _compare(coords, block, r)


def test_two_volumes_with_different_shapes_and_offsets():
    a = si.raster_coords((8, 8, 16))[si.packing_permutation((8, 8, 16), "random", seed=1)]
    b = si.raster_coords((16, 8, 8))[si.packing_permutation((16, 8, 8), "morton")] + np.array([100, -50, 7])
    coords = torch.from_numpy(np.stack([a, b]).astype(np.int32))
    _compare(coords, (4, 4, 4), 1)


def _expect_coords_error(coords, block, r, words):
    with pytest.raises(p3.Pack3DError) as e:
        p3.build_index(coords.to(DEV), block, r)
    assert e.value.status == p3.E_COORDS
    for wd in words:
        assert wd in str(e.value)


def test_geometry_errors():
    c = si.raster_coords((4, 4, 8))
    dup = c.copy()
    dup[40] = dup[12]                  # point 12 twice, interior point 40 missing
    _expect_coords_error(torch.from_numpy(dup[None]), (2, 2, 2), 1, ["duplicate", "local index 40"])
    out = c.copy()
    out[3] = (9, 0, 0)                 # outside: holes in the bounding box
    _expect_coords_error(torch.from_numpy(out[None]), (2, 2, 2), 1, ["fill"])
    nd = si.raster_coords((4, 4, 6))   # 6 not divisible by 4
    _expect_coords_error(torch.from_numpy(nd[None]), (2, 2, 4), 1, ["divisible"])
    two = np.stack([c, dup])
    _expect_coords_error(torch.from_numpy(two), (2, 2, 2), 1, ["volume 1"])
    # the oracle agrees on every case
    for bad, reason in ((dup, "duplicate"), (out, "grid")):
        with pytest.raises(oracle.CoordsError) as e:
            oracle.build_index(bad[None], (2, 2, 2), 1)
        assert e.value.reason == reason
