"""GPU position modes (controls) against the fp64 oracle.

"Geometry Matters in Packed 3D Attention" (abstract): packed-position encodings break
under repacking, axial grid-coordinate RoPE does not.  The library's position_mode swaps
only the rotation of the same operator: "packed1d" (1D RoPE on the packed position) and
"none" (no rotation), next to the default "axial".  Tolerances: max-abs 1e-5 (fp32
inputs), 2e-2 (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import DEV, TOL, max_err, sample_blocks, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (grid, block, r, heads, head_dim, packing, batch, dtype)
    ((8, 8, 16), (4, 4, 4), 1, 2, 96, "random", 2, torch.float32),
    ((8, 8, 16), (4, 4, 4), 1, 2, 96, "random", 2, torch.bfloat16),   # Dp 96 bf16 kernels
    ((4, 12, 8), (2, 3, 4), 1, 3, 12, "morton", 1, torch.float32),    # bvol 24, Dp 32
    ((8, 8, 8), (2, 2, 4), 2, 2, 66, "raster", 1, torch.bfloat16),    # Dp 96 with padding, r = 2
]


def run(w, dtype, mode, with_grad=False, packing=None):
    x = si.make_inputs(w, dtype, with_grad=with_grad, **({} if packing is None else {"packing": packing}))
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], position_mode=mode)
    grads = None
    if with_grad:
        grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], position_mode=mode)
    torch.cuda.synchronize()
    return x, ix, out, lse, grads


@pytest.mark.parametrize("grid,block,r,heads,d,packing,batch,dtype", CASES)
@pytest.mark.parametrize("mode", ["packed1d", "none"])
def test_forward_backward_match_oracle(grid, block, r, heads, d, packing, batch, dtype, mode):
    w = si.small_workload(grid=grid, block=block, radius=r, heads=heads, head_dim=d, packing=packing,
                          batch=batch, seed=41)
    say(f"position {mode} {grid} {block} r={r} D={d} {packing} {dtype}")
    x, _, out, lse, grads = run(w, dtype, mode, with_grad=True)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], block, r, position_mode=mode)
    assert max_err(out, o_ref) < TOL[dtype]
    assert max_err(lse, l_ref) < TOL[dtype]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], block, r, position_mode=mode)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        err = max_err(g, rr)
        assert err < TOL[dtype], (name, err)


def test_packed1d_rotation_intermediates():
    """Q~ = R_1D(packed position) q in canonical order, against the oracle's rope_1d."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, packing="random", seed=42)
    dtype = torch.float32
    x = si.make_inputs(w, dtype)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    attn = p3.make_attn(dtype, w.heads, w.head_dim, position_mode="packed1d")
    ws = torch.empty(p3.workspace_bytes(ix, attn), dtype=torch.uint8, device=DEV)
    p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], workspace=ws, position_mode="packed1d")
    torch.cuda.synchronize()
    views = p3.workspace_views(ix, (1, w.tokens, w.heads, w.head_dim), dtype, ws, position_mode="packed1d")
    perm = oracle.build_index(x["coords"].numpy(), w.block, w.radius)[0]["perm"]
    want = oracle.rope_1d(x["q"][0].double().numpy()[perm], perm)
    got = views["qrot"][0].float().cpu().numpy().transpose(1, 0, 2)
    assert np.abs(got - want).max() < 2e-6 * max(1.0, np.abs(want).max())


def test_packed1d_full_size_sampled_blocks():
    """65k launch in packed 1D mode (angle table of 65,536 rows); sampled query blocks."""
    w = si.WORKLOADS["65k"]
    dtype = torch.bfloat16
    say("position packed1d 65k")
    x, _, out, lse, _ = run(w, dtype, "packed1d")
    nb = tuple(g // b for g, b in zip(w.grid, w.block))
    blocks = sample_blocks(nb, count=6, seed=w.seed)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius, query_blocks=blocks,
                                  position_mode="packed1d")
    mask = ~np.isnan(o_ref)
    assert max_err(out, o_ref, mask) < TOL[dtype]
    assert max_err(lse, l_ref, ~np.isnan(l_ref)) < TOL[dtype]


def test_repacking_behaviour():
    """Bitwise-equivariant under repacking with axial RoPE and with no rotation; the outputs
    move with packed 1D RoPE (the failure mode of the abstract)."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, seed=43)
    dtype = torch.bfloat16
    res = {}
    for packing in ("raster", "random"):
        for mode in ("axial", "packed1d", "none"):
            x, _, out, _, _ = run(w, dtype, mode, packing=packing)
            inv = torch.argsort(x["perm"][0]).to(DEV)
            res[(packing, mode)] = out[0][inv]
    for mode in ("axial", "none"):
        assert torch.equal(res[("random", mode)], res[("raster", mode)]), mode
    diff = (res[("random", "packed1d")].float() - res[("raster", "packed1d")].float()).abs().max().item()
    assert diff > 5e-2


def test_autograd_wrapper_packed1d():
    w = si.small_workload(grid=(8, 8, 8), block=(2, 2, 4), heads=2, head_dim=48, packing="morton", seed=44)
    dtype = torch.float32
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    q, k, v = (xd[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = p3.attention(q, k, v, ix, xd["coords"], position_mode="packed1d")
    (o * xd["do"]).sum().backward()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius, position_mode="packed1d")
    for g, rr in zip((q.grad, k.grad, v.grad), ref):
        assert max_err(g, rr) < TOL[dtype]
