"""Host-side checks of the synthetic repacking task (sparse_local_global_amd.repacking): the
labeling rule against its definition written out voxel by voxel, and the packings as
permutations that move tokens without changing the physical volume or its labels."""
import numpy as np
import pytest
import torch

from sparse_local_global_amd import repacking as rp


def _labels_by_loops(cls, classes):
    z, y, x = cls.shape
    out = np.full(cls.shape, -1)
    for i in range(z):
        for j in range(y):
            for k in range(x):
                if i + 1 < z and j + 1 < y and k + 1 < x:
                    out[i, j, k] = cls[i + 1, j, k] + classes * cls[i, j + 1, k] + classes ** 2 * cls[i, j, k + 1]
    return out


@pytest.mark.parametrize("grid,classes", [((4, 5, 6), 4), ((3, 3, 3), 3), ((2, 7, 4), 5)])
def test_labeling_rule_matches_its_definition(grid, classes):
    rng = np.random.default_rng(1)
    cls = rng.integers(0, classes, size=grid)
    got = rp.labels_from_grid(torch.from_numpy(cls), classes).numpy()
    assert np.array_equal(got, _labels_by_loops(cls, classes))


def test_labels_unlabelled_only_on_high_faces():
    cls = torch.zeros(4, 4, 4, dtype=torch.int64)
    lab = rp.labels_from_grid(cls, 4)
    assert (lab[:3, :3, :3] == 0).all()
    assert (lab[3] == -1).all() and (lab[:, 3] == -1).all() and (lab[:, :, 3] == -1).all()


@pytest.mark.parametrize("packing", rp.PACKINGS)
def test_packings_are_permutations_that_keep_the_volume(packing):
    cfg = rp.TaskConfig(grid=(8, 8, 8), batch=2)
    rng = np.random.default_rng(3)
    cls, lab, coords, perms = rp.make_batch(cfg, rng, packing, 2, "cpu")
    rc = rp.raster_coords(cfg.grid)
    for v in range(2):
        assert sorted(perms[v].tolist()) == list(range(cfg.tokens))
        # every token keeps its coordinates, class and label: scattering back to raster order
        # gives a full grid whose labels follow the rule from its classes
        raster_cls = torch.empty(cfg.tokens, dtype=torch.int64)
        raster_cls[perms[v]] = cls[v]
        raster_lab = torch.empty(cfg.tokens, dtype=torch.int64)
        raster_lab[perms[v]] = lab[v]
        assert np.array_equal(coords[v].numpy(), rc[perms[v].numpy()])
        want = rp.labels_from_grid(raster_cls.view(*cfg.grid), cfg.classes).view(-1)
        assert torch.equal(raster_lab, want)


def test_block_and_morton_orders():
    grid, block = (4, 4, 4), (2, 2, 2)
    bo = rp.block_order(grid, block)
    rc = rp.raster_coords(grid)
    # the first 8 tokens of block order are the first 2x2x2 block
    assert {tuple(c) for c in rc[bo[:8]]} == {(z, y, x) for z in range(2) for y in range(2) for x in range(2)}
    mo = rp.morton_order(grid)
    # Morton order of a 2^k cube also visits aligned 2x2x2 cells one after another
    assert {tuple(c) for c in rc[mo[:8]]} == {(z, y, x) for z in range(2) for y in range(2) for x in range(2)}
    assert tuple(rc[mo[1]]) == (0, 0, 1) and tuple(rc[mo[2]]) == (0, 1, 0) and tuple(rc[mo[4]]) == (1, 0, 0)
