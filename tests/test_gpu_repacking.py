"""The synthetic repacking experiment on the GPU (sparse_local_global_amd.repacking): models
trained on raster-packed volumes, evaluated on Morton, block-contiguous and random packings
of fresh volumes ("Geometry Matters in Packed 3D Attention", abstract: encodings indexed by
the packed position fit the training layout and fail under repacking; axial RoPE on grid
coordinates does not).

The axial model's predictions must permute exactly with the tokens: every part of it is
per token except the operator, which is equivariant to repacking, so the same physical
voxel gets the same prediction under every packing.  The packed-position controls must
fit the training layout and fall towards chance (1/8) under repacking."""
import pytest
import torch

from sparse_local_global_amd import repacking as rp
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu

CFG = rp.TaskConfig()


def _evaluate_all(model):
    return {pk: rp.evaluate(model, CFG, pk) for pk in rp.PACKINGS}


def test_axial_model_is_exact_under_repacking():
    say("repacking: training the axial model")
    model, steps = rp.train(CFG, "axial")
    say(f"  fitted after {steps} steps")
    res = _evaluate_all(model)
    acc_r, pred_r, _ = res["raster"]
    assert acc_r >= 0.99
    for pk in ("morton", "block", "random"):
        acc, pred, _ = res[pk]
        say(f"  {pk}: accuracy {acc:.4f}")
        assert torch.equal(pred, pred_r), pk     # the same voxel, the same prediction
        assert acc == acc_r, pk


@pytest.mark.parametrize("mechanism", ["packed1d", "learned"])
def test_packed_position_controls_collapse_under_repacking(mechanism):
    say(f"repacking: training the {mechanism} control")
    model, steps = rp.train(CFG, mechanism)
    say(f"  fitted after {steps} steps")
    res = _evaluate_all(model)
    assert res["raster"][0] >= 0.99                  # the training layout is solved
    for pk in ("morton", "block", "random"):
        acc = res[pk][0]
        say(f"  {pk}: accuracy {acc:.4f}")
        assert acc < 0.5, pk                         # chance is 1/8
    assert res["random"][0] < 0.25
