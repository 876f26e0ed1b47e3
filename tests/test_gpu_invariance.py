"""Invariances of the method checked on the GPU at the 65k workload (2 volumes of 32x32x64,
8 heads, D = 96, 4x4x4 blocks, bf16), in the launch configuration the benchmark times.

"Geometry Matters in Packed 3D Attention" (abstract): attention is indexed by the true
grid coordinates, never by the packed position, so the same volume stored in raster,
Morton, block-contiguous or random order must give the same outputs and gradients token
for token; and every logit depends on coordinate differences only, so a global shift of
the coordinates changes nothing.  The kernels work in a canonical order derived from the
coordinates and sum in fixed orders, so both hold bitwise, and so does a repeated call.
"""
import pytest
import torch

import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import say, to_dev

pytestmark = pytest.mark.gpu

W = si.WORKLOADS["65k"]


def _step_in_raster_order(packing, shift=(0, 0, 0), repeat=1):
    """Forward and backward on the 65k inputs stored in `packing` order; results returned in
    raster order (token at packed position p of volume v is raster token perm[v, p])."""
    x = si.make_inputs(W, torch.bfloat16, packing=packing, with_grad=True, shift=shift)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], W.block, W.radius)
    runs = []
    for _ in range(repeat):
        out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"])
        dq, dk, dv = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"])
        torch.cuda.synchronize()
        inv = [torch.argsort(x["perm"][v]).to(xd["q"].device) for v in range(W.batch)]
        res = {}
        for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
            res[name] = torch.stack([t[v][inv[v]] for v in range(W.batch)])
        res["lse"] = torch.stack([lse[v][:, inv[v]] for v in range(W.batch)])
        runs.append(res)
    return runs


def _assert_bitwise(a, b, what):
    for name in ("out", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), f"{what}: {name} differs"


def test_repeated_calls_are_bitwise_equal():
    say("65k: repeated forward + backward")
    r1, r2 = _step_in_raster_order("random", repeat=2)
    _assert_bitwise(r1, r2, "second call")
    assert all(torch.isfinite(r1[n]).all() for n in ("out", "lse", "dq", "dk", "dv"))


def test_repacking_and_shift_change_nothing():
    ref = _step_in_raster_order("raster")[0]
    for packing in ("morton", "block", "random"):
        say(f"65k: {packing} packing")
        _assert_bitwise(_step_in_raster_order(packing)[0], ref, f"{packing} packing")
    say("65k: shifted coordinates")
    _assert_bitwise(_step_in_raster_order("random", shift=(7, -300, 1 << 20))[0], ref, "global shift")
