"""GPU path at its size limits and on degenerate geometries, against the fp64 oracle.

Limits of the attention kernels (each rejected beyond with PACK3D_E_UNSUPPORTED):
16384 blocks per volume (the per-query-block summary mask is held in LDS), 1024 tokens
per block, local radius 3.  The degenerate geometries are the ones the locality rule of
"Geometry Matters in Packed 3D Attention" (block-granular locality, Chebyshev radius r,
one summary per distant block) reduces on: a volume that is a single block (no
summaries), a radius that covers the whole block grid (dense attention), and volumes one
token thick along one or two axes.

At the block-count maximum the oracle computes o, lse and dq on sampled query blocks.
dk and dv need every query there (minutes of fp64 work per head), so the oracle's
gradients of one head on the tokens of sampled blocks are stored by
tests/golden/make_limit_gradients.py and compared element by element, and over all
tokens dk and dv are held to two exact identities of the method (each query's weights
over keys and summaries sum to one, and a block mean hands a summary's gradient to its
members in full):
    sum_j dv_j = sum_i dO_i            and        sum_j R_j dk_j = 0
per (volume, head, channel), R_j the token's rotation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.dense_ref import torch_axial_rope
from tests.gpu_cases import DEV, TOL, max_err, sample_blocks, say, to_dev

pytestmark = pytest.mark.gpu

MAX_BLOCKS = 16384
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "limit_gradients.json")


def _run(w, x, with_summaries=True):
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base,
                          with_summaries=with_summaries)
    grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"],
                        rope_base=w.rope_base, with_summaries=with_summaries)
    torch.cuda.synchronize()
    return ix, out, lse, grads


# Conservation bounds, relative to sum_i |dO_i| per (head, channel).  bf16: the products
# P dO and dS Q~ take bf16 operands (relative rounding <= 2^-9 each) and dk, dv are stored
# in bf16 (another 2^-9), so the worst-case sum of errors stays below 2^-7 of the sum of the
# magnitudes involved.  fp32: the same argument with fp32 rounding and the kernels' fp32
# exponent, bounded by 1e-5.
CONS_REL = {torch.float32: 1e-5, torch.bfloat16: 2.0 ** -7}


@pytest.mark.parametrize("dtype,heads,d", [(torch.float32, 1, 12), (torch.bfloat16, 2, 96)])
def test_maximum_blocks_per_volume(dtype, heads, d):
    """16384 blocks of 2x2x2 tokens in one volume (131072 tokens)."""
    w = si.small_workload(grid=(32, 64, 64), block=(2, 2, 2), radius=1, heads=heads, head_dim=d,
                          packing="random", seed=61)
    nb = (16, 32, 32)
    assert int(np.prod(nb)) == MAX_BLOCKS
    say(f"maximum block count {dtype} H={heads} D={d}")
    x = si.make_inputs(w, dtype, with_grad=True)
    x["do"] = (x["do"].float() + 0.75).to(dtype)   # a mean offset makes the dv identity sensitive
    ix, out, lse, (dq, dk, dv) = _run(w, x)
    assert ix.tables()["nblk"] == MAX_BLOCKS
    blocks = sample_blocks(nb, count=8, seed=w.seed)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius, query_blocks=blocks)
    mask = ~np.isnan(o_ref)
    assert mask.sum() == len(blocks) * 8 * heads * d
    assert max_err(out, o_ref, mask) < TOL[dtype]
    assert max_err(lse, l_ref, ~np.isnan(l_ref)) < TOL[dtype]
    dq_ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius,
                             query_blocks=blocks)[0]
    qmask = ~np.isnan(dq_ref)
    assert qmask.sum() == mask.sum()
    assert max_err(dq, dq_ref, qmask) < TOL[dtype]
    for g in (out, lse, dq, dk, dv):
        assert torch.isfinite(g).all()
    # every gradient of one head element by element on the tokens of sampled blocks, against
    # the oracle's values stored by tests/golden/make_limit_gradients.py (minutes of fp64 work
    # per head, run once on the CPU)
    golden = json.load(open(GOLDEN))
    assert tuple(golden["grid"]) == w.grid and tuple(golden["block"]) == w.block and golden["seed"] == w.seed
    case = golden["cases"]["fp32_d12" if dtype == torch.float32 else "bf16_d96"]
    assert (case["heads"], case["head_dim"]) == (heads, d)
    h, tok = case["head"], torch.tensor(case["tokens"])
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = g[0][tok.to(DEV), h].double().cpu().numpy()
        err = float(np.abs(got - np.asarray(case[name])).max())
        say(f"  {name} on {len(tok)} stored tokens of head {h}: max err {err:.3e}")
        assert err < TOL[dtype], (name, err)
    # identities for dk and dv over all 131072 tokens
    do64 = x["do"][0].double()
    scale = do64.abs().sum(0)                                            # [H, D]
    gap = dv[0].double().cpu().sum(0) - do64.sum(0)
    assert (gap.abs() <= CONS_REL[dtype] * scale).all(), float((gap.abs() / scale).max())
    c = x["coords"][0].long()
    rel = c - c.min(0).values
    rot = torch_axial_rope(dk[0].double().cpu(), rel, w.rope_base).sum(0)
    assert (rot.abs() <= CONS_REL[dtype] * scale).all(), float((rot.abs() / scale).max())


def test_blocks_beyond_limit_are_rejected():
    """16896 blocks per volume: the index builds, the attention entry points refuse it."""
    w = si.small_workload(grid=(32, 64, 66), block=(2, 2, 2), radius=1, heads=1, head_dim=12, seed=62)
    x = to_dev(si.make_inputs(w, torch.float32, with_grad=True))
    say("block count beyond the limit")
    for ragged in (False, True):
        ix = p3.build_index(x["coords"], w.block, 1, ragged=ragged)
        assert ix.tables()["nblk"] == 16 * 32 * 33
        with pytest.raises(p3.Pack3DError) as e:
            p3.forward(ix, x["q"], x["k"], x["v"], x["coords"])
        assert e.value.status == p3.E_UNSUPPORTED and "blocks per volume" in str(e.value)
        out = torch.zeros_like(x["q"])
        lse = torch.zeros((1, 1, w.tokens), dtype=torch.float32, device=DEV)
        with pytest.raises(p3.Pack3DError) as e:
            p3.backward(ix, x["q"], x["k"], x["v"], x["coords"], out, lse, x["do"])
        assert e.value.status == p3.E_UNSUPPORTED


def _full_compare(w, dtype, with_summaries=True):
    x = si.make_inputs(w, dtype, with_grad=True)
    _, out, lse, grads = _run(w, x, with_summaries)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius,
                                  with_summaries=with_summaries)
    assert max_err(out, o_ref) < TOL[dtype]
    assert max_err(lse, l_ref) < TOL[dtype]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius,
                          with_summaries=with_summaries)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        err = max_err(g, rr)
        assert err < TOL[dtype], (name, err)


DTYPES = [(torch.float32, 48), (torch.bfloat16, 96)]


@pytest.mark.parametrize("dtype,d", DTYPES)
def test_maximum_block_tokens(dtype, d):
    """1024-token blocks (8x8x16): 16 query tiles per block, 7 summaries per query at r = 0."""
    w = si.small_workload(grid=(16, 16, 32), block=(8, 8, 16), radius=0, heads=2, head_dim=d,
                          packing="random", seed=63)
    say(f"1024-token blocks {dtype}")
    _full_compare(w, dtype)


GEOMETRIES = [
    # (grid, block, r, batch, label)
    ((2, 2, 2), (2, 2, 2), 1, 2, "two 8-token volumes, one block each"),
    ((4, 4, 4), (4, 4, 4), 0, 1, "one 64-token block, r = 0"),
    ((4, 8, 8), (2, 2, 2), 3, 1, "radius covers the block grid: dense"),
    ((1, 16, 32), (1, 2, 4), 1, 1, "one token thick along z"),
    ((1, 1, 256), (1, 1, 8), 2, 1, "a line of tokens along x"),
    ((16, 1, 1), (8, 1, 1), 0, 1, "a line of two blocks along z"),
]


@pytest.mark.parametrize("grid,block,r,batch,label", GEOMETRIES)
@pytest.mark.parametrize("dtype,d", DTYPES)
def test_degenerate_geometries(grid, block, r, batch, label, dtype, d):
    w = si.small_workload(grid=grid, block=block, radius=r, heads=2, head_dim=d, packing="random",
                          batch=batch, seed=64)
    say(f"degenerate geometry: {label} {dtype}")
    _full_compare(w, dtype)


def test_dense_case_ignores_summaries_switch():
    """When the radius covers every block there are no summaries: both settings agree bitwise."""
    w = si.small_workload(grid=(4, 8, 8), block=(2, 2, 2), radius=3, heads=2, head_dim=96, seed=65)
    x = si.make_inputs(w, torch.bfloat16, with_grad=True)
    say("dense case, summaries on and off")
    _, o1, l1, g1 = _run(w, x, True)
    _, o2, l2, g2 = _run(w, x, False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    assert math.isfinite(float(l1.max()))
