"""GPU forward (K1 RoPE/gather, K2 pooling, K3 fused attention) against the fp64 oracle.

Tolerances: max-abs 1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32
accumulation, on o; lse is held to the same bounds.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import DEV, TOL, gpu_forward, max_err, sample_blocks, say, to_dev

pytestmark = pytest.mark.gpu


def _canonical(x, ix_ref, v):
    return x[v][ix_ref[v]["perm"]]


# 48-token blocks: the RoPE / pooling pass stages tokens 32 at a time, so each block ends
# in a partial chunk whose tokens must be gathered, rotated and pooled like the others
INTERMEDIATE_CASES = {
    "tiny": si.WORKLOADS["tiny"],
    "16k": si.WORKLOADS["16k"],
    "bvol48": si.small_workload(grid=(8, 8, 12), block=(4, 4, 3), heads=2, head_dim=96, packing="random", seed=23),
}


@pytest.mark.parametrize("name,dtype", [("tiny", torch.float32), ("16k", torch.bfloat16),
                                        ("bvol48", torch.float32), ("bvol48", torch.bfloat16)])
def test_intermediates_rope_and_pooling(name, dtype):
    w = INTERMEDIATE_CASES[name]
    say(f"intermediates {name} {dtype}")
    x, ix, out, lse, ws = gpu_forward(w, dtype)
    views = p3.workspace_views(ix, (w.batch, w.tokens, w.heads, w.head_dim), dtype, ws, w.rope_base)
    ref = oracle.build_index(x["coords"].numpy(), w.block, w.radius)
    d = w.head_dim
    tol = 2e-6 if dtype == torch.float32 else 2e-2
    for v in range(w.batch):
        perm = ref[v]["perm"]
        rel = x["coords"][v].numpy()[perm] - ref[v]["origin"]      # origin-relative angles
        qc = x["q"][v].double().numpy()[perm]
        kc = x["k"][v].double().numpy()[perm]
        vc = x["v"][v].double().numpy()[perm]
        qr = oracle.rope(qc, rel, w.rope_base)
        kr = oracle.rope(kc, rel, w.rope_base)
        gq = views["qrot"][v].float().cpu().numpy().transpose(1, 0, 2)
        gk = views["krot"][v].float().cpu().numpy().transpose(1, 0, 2)
        assert np.abs(gq[..., :d] - qr).max() < tol * max(1.0, np.abs(qr).max())
        assert np.abs(gk[..., :d] - kr).max() < tol * max(1.0, np.abs(kr).max())
        assert (gq[..., d:] == 0).all() and (gk[..., d:] == 0).all()
        bvol, nblk = ref[v]["bvol"], ref[v]["nblk"]
        kbar = oracle.pool_blocks(kr, bvol)                           # [nblk, H, D]
        vbar = oracle.pool_blocks(vc, bvol)
        gkb = views["kbar"][v].float().cpu().numpy()                  # [H, nblkp, Dp]
        gvb = views["vbar"][v].float().cpu().numpy()                  # [H, nblkp, Dp]
        assert np.abs(gkb[:, :nblk, :d] - kbar.transpose(1, 0, 2)).max() < tol
        assert np.abs(gvb[:, :nblk, :d] - vbar.transpose(1, 0, 2)).max() < tol
        assert (gkb[:, nblk:] == 0).all() and (gvb[:, nblk:] == 0).all()
        gv = views["vrow"][v].float().cpu().numpy().transpose(1, 0, 2)  # [N, H, Dp]
        assert np.array_equal(gv[..., :d], vc) and (gv[..., d:] == 0).all()   # V is copied exactly


CASES = [
    # (grid, block, r, heads, head_dim, packing, batch, dtype)
    ((8, 8, 8), (2, 2, 2), 1, 2, 48, "raster", 1, torch.float32),     # bvol 8: ragged local tiles
    ((8, 8, 16), (4, 4, 4), 1, 2, 96, "random", 2, torch.float32),
    ((8, 8, 16), (4, 4, 4), 1, 2, 96, "random", 2, torch.bfloat16),
    ((8, 16, 16), (4, 8, 8), 1, 2, 96, "block", 1, torch.bfloat16),  # 256-token blocks: 4 query tiles
    ((4, 12, 8), (2, 3, 4), 1, 3, 12, "morton", 1, torch.float32),   # bvol 24, Dp 32
    ((8, 8, 8), (2, 2, 4), 2, 2, 120, "random", 1, torch.bfloat16),  # Dp 128, r = 2
    ((8, 8, 8), (4, 4, 4), 0, 1, 66, "random", 1, torch.float32),    # r = 0, Dp 96 with padding
    ((4, 8, 8), (2, 2, 2), 3, 2, 24, "raster", 1, torch.bfloat16),   # r = 3 (slots 343)
    ((8, 8, 8), (2, 2, 4), 1, 2, 90, "morton", 1, torch.bfloat16),   # Dp 96 with padding, bvol 16
    # blocks of 40, 48 and 56 tokens: the RoPE / pooling pass stages 32 tokens at a time,
    # so the last chunk of each block is partial
    ((8, 8, 12), (4, 4, 3), 1, 2, 96, "random", 1, torch.float32),   # bvol 48
    ((8, 8, 12), (4, 4, 3), 1, 2, 96, "random", 1, torch.bfloat16),  # bvol 48
    ((4, 8, 10), (2, 4, 5), 1, 2, 48, "morton", 1, torch.bfloat16),  # bvol 40, Dp 64
    ((4, 8, 14), (2, 4, 7), 1, 2, 96, "block", 1, torch.float32),    # bvol 56
]


@pytest.mark.parametrize("grid,block,r,heads,d,packing,batch,dtype", CASES)
@pytest.mark.parametrize("with_s", [True, False])
def test_forward_matches_oracle_small(grid, block, r, heads, d, packing, batch, dtype, with_s):
    w = si.small_workload(grid=grid, block=block, radius=r, heads=heads, head_dim=d, packing=packing,
                          batch=batch, seed=17)
    say(f"forward {grid} {block} r={r} H={heads} D={d} {packing} B={batch} {dtype} summaries={with_s}")
    x, ix, out, lse, _ = gpu_forward(w, dtype, with_summaries=with_s)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], block, r, with_summaries=with_s)
    assert max_err(out, o_ref) < TOL[dtype]
    assert max_err(lse, l_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32])
def test_forward_tiny_workload(dtype):
    w = si.WORKLOADS["tiny"]
    say("forward tiny workload")
    x, ix, out, lse, _ = gpu_forward(w, dtype)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius)
    assert max_err(out, o_ref) < TOL[dtype] and max_err(lse, l_ref) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_forward_16k_workload_full(dtype):
    w = si.WORKLOADS["16k"]
    say(f"forward 16k {dtype}")
    x, ix, out, lse, _ = gpu_forward(w, dtype)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius)
    assert max_err(out, o_ref) < TOL[dtype] and max_err(lse, l_ref) < TOL[dtype]


@pytest.mark.parametrize("name,with_s", [("65k", True), ("65k", False), ("524k", True)])
def test_forward_full_size_sampled_blocks(name, with_s):
    """Full-size launch (the benchmark's configuration); the oracle computes sampled query blocks."""
    w = si.WORKLOADS[name]
    dtype = torch.bfloat16
    say(f"forward {name} summaries={with_s}")
    x, ix, out, lse, _ = gpu_forward(w, dtype, with_summaries=with_s)
    nb = tuple(g // b for g, b in zip(w.grid, w.block))
    blocks = sample_blocks(nb, count=10, seed=w.seed)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius,
                                  with_summaries=with_s, query_blocks=blocks)
    mask = ~np.isnan(o_ref)
    assert mask.sum() == w.batch * len(blocks) * int(np.prod(w.block)) * w.heads * w.head_dim
    assert max_err(out, o_ref, mask) < TOL[dtype]
    lmask = ~np.isnan(l_ref)
    assert max_err(lse, l_ref, lmask) < TOL[dtype]
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_deterministic_repacking_and_shift_bitwise():
    """Two runs are bitwise equal; repacking permutes outputs bitwise; a global shift changes nothing."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, packing="random", seed=3)
    dtype = torch.bfloat16
    _, _, o1, l1, _ = gpu_forward(w, dtype)
    _, _, o2, l2, _ = gpu_forward(w, dtype)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    outs = {}
    for packing in si.PACKINGS:
        x, _, o, l, _ = gpu_forward(w, dtype, packing=packing)
        inv = torch.argsort(x["perm"][0]).to(DEV)
        outs[packing] = (o[0][inv], l[0][:, inv])
    for packing in si.PACKINGS[1:]:
        assert torch.equal(outs[packing][0], outs["raster"][0]), packing
        assert torch.equal(outs[packing][1], outs["raster"][1]), packing
    x, _, o3, l3, _ = gpu_forward(w, dtype, shift=(5, -13, 1001))
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_poisoned_buffers_are_never_read():
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=48, packing="random", seed=8)
    dtype = torch.float32
    x, ix, o1, l1, _ = gpu_forward(w, dtype)
    xd = to_dev(x)
    attn = p3.make_attn(dtype, w.heads, w.head_dim)
    ws = torch.full((p3.workspace_bytes(ix, attn) // 4,), float("nan"), device=DEV).view(torch.uint8)
    out = torch.full_like(xd["q"], float("nan"))
    lse = torch.full((1, 2, w.tokens), float("nan"), device=DEV)
    p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, o1) and torch.equal(lse, l1)


def test_forward_errors():
    w = si.small_workload(grid=(4, 4, 8), block=(2, 2, 2), heads=1, head_dim=12, seed=1)
    x = to_dev(si.make_inputs(w, torch.float32))
    ix = p3.build_index(x["coords"], w.block, 1)
    attn = p3.make_attn(torch.float32, 1, 12)
    ws = torch.empty(p3.workspace_bytes(ix, attn), dtype=torch.uint8, device=DEV)
    with pytest.raises(p3.Pack3DError) as e:
        p3.forward(ix, x["q"], x["k"], x["v"], x["coords"], workspace=ws[:100])
    assert e.value.status == p3.E_WORKSPACE
    bad = torch.zeros(1, w.tokens, 1, 8, device=DEV)
    with pytest.raises(p3.Pack3DError) as e:
        p3.forward(ix, bad, bad, bad, x["coords"])
    assert e.value.status == p3.E_UNSUPPORTED
    with pytest.raises(p3.Pack3DError) as e:
        p3.forward(ix, x["q"].half(), x["k"].half(), x["v"].half(), x["coords"])
    assert e.value.status == p3.E_UNSUPPORTED
    # buffers a caller hands in must have the sizes the index implies: refused before any launch
    lse = torch.empty((1, 1, w.tokens), dtype=torch.float32, device=DEV)
    for kw in (dict(out=torch.empty_like(x["q"])[:, :-1]),
               dict(out=torch.empty_like(x["q"]).transpose(2, 3)),
               dict(lse=lse.double()),
               dict(lse=lse[:, :, :-1]),
               dict(workspace=ws.view(torch.float32))):
        with pytest.raises(p3.Pack3DError) as e:
            p3.forward(ix, x["q"], x["k"], x["v"], x["coords"], **kw)
        assert e.value.status == p3.E_INVALID, kw
    with pytest.raises(p3.Pack3DError) as e:
        p3.forward(ix, x["q"], x["k"], x["v"], x["coords"][:, :-1].contiguous())
    assert e.value.status == p3.E_INVALID


@pytest.mark.parametrize("scale", [3.0, 6.0])
def test_large_logits_exact_operands(scale):
    """Logits spread over tens to hundreds of units (lse up to about 190 at scale 6), so later
    tiles overtake the running reference maximum by far more than 2^8 and the forward takes
    its exact-maximum rescaling branch mid-stream, not only on the first tile.  Position mode
    "none" keeps the rotated operands equal to the bf16 inputs, so scores are exact products
    on both sides and the bf16 rounding of the weights is the only approximation.  Outputs and
    gradients grow with the inputs (|o| reaches about 8 at scale 3, where half a bf16 ulp is
    already 0.03), so they are held to 2e-2 of their largest reference magnitude; lse keeps
    the absolute bound."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), radius=1, heads=2, head_dim=96, packing="random",
                          seed=72, input_scale=scale)
    dtype = torch.bfloat16
    say(f"large logits scale={scale}")
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], position_mode="none")
    grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], position_mode="none")
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius, position_mode="none")
    assert max_err(out, o_ref) < TOL[dtype] * max(1.0, float(np.abs(o_ref).max()))
    assert max_err(lse, l_ref) < TOL[dtype]
    assert float(np.nanmax(l_ref)) > 15.0 * scale
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius, position_mode="none")
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        err = max_err(g, rr)
        assert err < TOL[dtype] * max(1.0, float(np.abs(rr).max())), (name, err, float(np.abs(rr).max()))
