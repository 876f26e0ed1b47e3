"""Pins of the oracle's index tables (block membership, canonical order, neighbours).

Geometry source: "Geometry Matters in Packed 3D Attention", abstract (contiguous
3D blocks, exact local neighbourhood).  Readings: block-granular locality with
Chebyshev radius r in block units, truncated at the volume edge; block ids
raster over the block grid; neighbour slots raster over (dz, dy, dx); -1
outside the grid.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _per_axis_pairs(nb, r):
    # number of (query, neighbour) block-coordinate pairs along one axis
    return sum(min(b + r, nb - 1) - max(b - r, 0) + 1 for b in range(nb))


def test_block_pair_totals_match_closed_form_fixture():
    """Sum over blocks of the local-set size = product of per-axis pair counts."""
    with open(os.path.join(GOLDEN, "block_pair_totals.json")) as f:
        fixture = json.load(f)
    for case in fixture["cases"]:
        grid, block, r = case["grid"], case["block"], case["radius"]
        nb = [g // b for g, b in zip(grid, block)]
        closed = int(np.prod([_per_axis_pairs(n, r) for n in nb]))
        assert closed == case["pairs"]
        ix = oracle.build_index(si.raster_coords(grid)[None], block, r)[0]
        assert int((ix["nbr"] >= 0).sum()) == case["pairs"]


@pytest.mark.parametrize("grid,block,r", [((4, 6, 8), (2, 2, 2), 1), ((6, 4, 4), (2, 1, 2), 2),
                                          ((8, 8, 8), (2, 2, 2), 0), ((4, 4, 8), (4, 4, 4), 1)])
def test_neighbour_table_brute_force(grid, block, r):
    ix = oracle.build_index(si.raster_coords(grid)[None], block, r)[0]
    nb = [g // b for g, b in zip(grid, block)]
    coords = list(itertools.product(*[range(n) for n in nb]))  # raster over blocks
    offsets = list(itertools.product(range(-r, r + 1), repeat=3))
    for bid, bc in enumerate(coords):
        for s, off in enumerate(offsets):
            tgt = tuple(a + d for a, d in zip(bc, off))
            want = coords.index(tgt) if all(0 <= t < n for t, n in zip(tgt, nb)) else -1
            assert ix["nbr"][bid, s] == want
        local = {int(x) for x in ix["nbr"][bid] if x >= 0}
        cheb = {j for j, oc in enumerate(coords) if max(abs(a - b) for a, b in zip(oc, bc)) <= r}
        assert local == cheb


@pytest.mark.parametrize("packing", si.PACKINGS)
def test_canonical_order_and_permutation(packing):
    grid, block = (4, 6, 8), (2, 3, 2)
    perm = si.packing_permutation(grid, packing, block=block, seed=3)
    coords = si.raster_coords(grid)[perm] + np.array([5, -7, 2], dtype=np.int32)
    ix = oracle.build_index(coords[None], block, 1)[0]
    n = coords.shape[0]
    assert sorted(ix["perm"].tolist()) == list(range(n))
    assert np.array_equal(ix["canon"][ix["perm"]], np.arange(n))
    cp = coords[ix["perm"]] - coords.min(0)              # coordinates in canonical order
    bvol = int(np.prod(block))
    for blk in range(n // bvol):
        rows = cp[blk * bvol:(blk + 1) * bvol]
        bc = rows // np.array(block)
        assert (bc == bc[0]).all()                         # one block per contiguous run
        w = rows - bc * np.array(block)
        lin = (w[:, 0] * block[1] + w[:, 1]) * block[2] + w[:, 2]
        assert np.array_equal(lin, np.arange(bvol))        # raster inside the block
    # blocks themselves in raster order
    firsts = cp[::bvol] // np.array(block)
    nb = np.array(grid) // np.array(block)
    assert np.array_equal((firsts[:, 0] * nb[1] + firsts[:, 1]) * nb[2] + firsts[:, 2], np.arange(n // bvol))


def test_tables_follow_tokens_under_repacking():
    grid, block = (4, 4, 8), (2, 2, 2)
    base = oracle.build_index(si.raster_coords(grid)[None], block, 1)[0]
    for packing in ("morton", "block", "random"):
        perm = si.packing_permutation(grid, packing, block=block, seed=11)
        ix = oracle.build_index(si.raster_coords(grid)[perm][None], block, 1)[0]
        assert np.array_equal(ix["token_block"], base["token_block"][perm])
        assert np.array_equal(ix["canon"], base["canon"][perm])
        assert np.array_equal(ix["nbr"], base["nbr"])


def test_error_cases():
    c = si.raster_coords((4, 4, 4))
    bad = c.copy()
    bad[9] = (7, 0, 0)                                     # a point outside -> holes in the box
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(bad[None], (2, 2, 2), 1)
    assert e.value.reason == "grid"
    # a pure duplicate: point 12 appears twice (tokens 12 and 40) and point 40 is
    # missing; the bounding box still holds N points, so the duplicate is reported
    dup = c.copy()
    dup[[10, 30]] = dup[[30, 10]]
    dup[40] = dup[12]
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(dup[None], (2, 2, 2), 1)
    assert e.value.reason == "duplicate" and e.value.token == 40
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(si.raster_coords((4, 4, 6))[None], (4, 4, 4), 1)
    assert e.value.reason == "divisible"
    with pytest.raises(ValueError):
        oracle.build_index(c[None], (2, 2, 2), -1)
    with pytest.raises(ValueError):
        oracle.build_index(c[None], (2, 0, 2), 1)
    # second volume bad, first fine
    two = np.stack([c, bad])
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(two, (2, 2, 2), 1)
    assert e.value.volume == 1
