"""GPU ragged geometry and varlen batches against the fp64 oracle.

"Geometry Matters in Packed 3D Attention" (abstract): packed geometric data in general.
A volume is any set of distinct points (partial edge blocks, holes); volumes of a batch
may differ in shape and token count (flat [T, H, D] with offsets).  Tolerances: max-abs
1e-5 (fp32 inputs), 2e-2 (bf16 inputs, fp32 accumulation); tables bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import DEV, TOL, max_err, say

pytestmark = pytest.mark.gpu

CASES = [
    # grids, block, r, occupancy, heads, head_dim, dtype
    ([(9, 10, 13)], (4, 4, 4), 1, 0.75, 2, 96, torch.bfloat16),           # one block per tile
    ([(9, 10, 13)], (4, 4, 4), 1, 0.75, 2, 96, torch.float32),
    ([(7, 9, 11), (12, 5, 6)], (2, 2, 2), 1, 0.6, 2, 48, torch.float32),  # 8-token blocks, varlen
    ([(10, 7, 9), (5, 12, 8)], (2, 2, 6), 1, 0.8, 3, 12, torch.bfloat16), # 24-token blocks, Dp 32
    ([(8, 8, 16)], (4, 4, 4), 2, 0.5, 2, 66, torch.bfloat16),             # r = 2, padded head dim
    ([(13, 20, 18)], (4, 8, 8), 1, 0.85, 2, 96, torch.bfloat16),          # four tiles per block
]


def _inputs(grids, heads, d, dtype, occ, seed, with_grad=True, shifts=None):
    return si.make_ragged_inputs(grids, heads, d, dtype, occupancy=occ, seed=seed, with_grad=with_grad,
                                 shifts=shifts)


def _run(x, block, r, dtype, with_grad=True, mode="axial"):
    off = x["offsets"].tolist()
    xd = {k: v.to(DEV) for k, v in x.items() if k in ("q", "k", "v", "coords", "do")}
    ix = p3.build_index(xd["coords"], block, r, ragged=True, offsets=off)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], position_mode=mode)
    grads = None
    if with_grad:
        grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], position_mode=mode)
    torch.cuda.synchronize()
    return ix, out, lse, grads


@pytest.mark.parametrize("grids,block,r,occ,heads,d,dtype", CASES)
def test_forward_backward_match_oracle(grids, block, r, occ, heads, d, dtype):
    say(f"ragged {grids} {block} r={r} occ={occ} D={d} {dtype}")
    x = _inputs(grids, heads, d, dtype, occ, seed=71)
    off = x["offsets"].numpy()
    _, out, lse, grads = _run(x, block, r, dtype)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], block, r, ragged=True, offsets=off)
    assert max_err(out, o_ref) < TOL[dtype]
    assert max_err(lse, l_ref, ~np.isnan(l_ref)) < TOL[dtype]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], block, r, ragged=True, offsets=off)
    ix = oracle.build_index(x["coords"].numpy(), block, r, ragged=True, offsets=off)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        diff = np.abs(g.float().cpu().double().numpy() - rr)
        err = float(diff.max())
        t = int(np.unravel_index(diff.argmax(), diff.shape)[0])
        v = int(np.searchsorted(off, t, side="right") - 1)
        blk = ix[v]["token_block"][t - off[v]]
        assert err < TOL[dtype], (name, err, float(np.abs(rr).max()), float(np.abs(rr[t]).max()),
                                  int(ix[v]["count"][blk]))


def test_index_tables_bit_exact():
    x = _inputs([(7, 9, 11), (12, 5, 6), (3, 4, 17)], 1, 6, torch.float32, 0.55, seed=72, with_grad=False,
                shifts=[(0, 0, 0), (-5, 3, 100), (7, -2, -9)])
    off = x["offsets"].tolist()
    ix = p3.build_index(x["coords"].to(DEV), (2, 2, 2), 1, ragged=True, offsets=off)
    t = ix.tables()
    ref = oracle.build_index(x["coords"].numpy(), (2, 2, 2), 1, ragged=True, offsets=off)
    assert t["holes"] and t["ragged"] and t["nblk"] == max(rv["nblk"] for rv in ref)
    assert t["volume_offsets"].cpu().tolist() == off
    nc = t["nblk"] * 8
    for v, rv in enumerate(ref):
        a, b = off[v], off[v + 1]
        assert np.array_equal(t["token_block"][a:b].cpu().numpy(), rv["token_block"])
        assert np.array_equal(t["canon"][a:b].cpu().numpy(), rv["canon"])
        perm = t["perm"][v].cpu().numpy()
        n_own = rv["nblk"] * 8
        assert np.array_equal(perm[:n_own], rv["perm"]) and (perm[n_own:nc] == -1).all()
        cnt = t["block_count"][v].cpu().numpy()
        assert np.array_equal(cnt[:rv["nblk"]], rv["count"]) and (cnt[rv["nblk"]:] == 0).all()
        nbr = t["nbr"][v].cpu().numpy()
        assert np.array_equal(nbr[:rv["nblk"]], rv["nbr"]) and (nbr[rv["nblk"]:] == -1).all()
        origin, extent = ix.geometry(v)
        assert origin == tuple(rv["origin"]) and extent == tuple(rv["extent"])


def test_measure_blocks():
    x = _inputs([(7, 9, 11), (12, 5, 6)], 1, 6, torch.float32, 0.5, seed=73, with_grad=False)
    off = x["offsets"].tolist()
    n = p3.measure_blocks(x["coords"].to(DEV), (2, 2, 4), offsets=off)
    assert n == max(4 * 5 * 3, 6 * 3 * 2)


def test_full_grid_ragged_flag_bitwise_same():
    """A full divisible grid through the ragged path has no empty slot: same kernels, same bits."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, packing="random", seed=74)
    x = si.make_inputs(w, torch.bfloat16, with_grad=True)
    xd = {k: v.to(DEV) for k, v in x.items()}
    res = []
    for ragged in (False, True):
        ix = p3.build_index(xd["coords"], w.block, w.radius, ragged=ragged)
        assert not ix.tables()["holes"]
        out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"])
        g = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"])
        res.append((out, lse) + tuple(g))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_repacking_bitwise_and_deterministic():
    x = _inputs([(9, 10, 13)], 2, 96, torch.bfloat16, 0.7, seed=75)
    _, out, lse, g = _run(x, (4, 4, 4), 1, torch.bfloat16)
    _, out2, lse2, g2 = _run(x, (4, 4, 4), 1, torch.bfloat16)
    for a, b in zip((out, lse) + tuple(g), (out2, lse2) + tuple(g2)):
        assert torch.equal(a, b)
    p = torch.from_numpy(np.random.default_rng(3).permutation(x["q"].shape[0]))
    y = dict(x)
    for k in ("q", "k", "v", "coords", "do"):
        y[k] = x[k][p].contiguous()
    _, out3, lse3, g3 = _run(y, (4, 4, 4), 1, torch.bfloat16)
    pd = p.to(DEV)
    assert torch.equal(out3, out[pd]) and torch.equal(lse3, lse[:, :, pd])
    for a, b in zip(g3, g):
        assert torch.equal(a, b[pd])


def test_packed1d_mode_on_ragged_batch():
    x = _inputs([(7, 9, 11), (12, 5, 6)], 2, 48, torch.float32, 0.6, seed=76)
    off = x["offsets"].numpy()
    _, out, lse, grads = _run(x, (2, 2, 2), 1, torch.float32, mode="packed1d")
    o_ref, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], (2, 2, 2), 1, ragged=True, offsets=off,
                              position_mode="packed1d")
    assert max_err(out, o_ref) < TOL[torch.float32]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], (2, 2, 2), 1, ragged=True, offsets=off,
                          position_mode="packed1d")
    for g, rr in zip(grads, ref):
        assert max_err(g, rr) < TOL[torch.float32]


def test_geometry_errors():
    c = torch.tensor([[0, 0, 0], [1, 1, 1], [0, 0, 0], [3, 2, 1]], dtype=torch.int32)
    with pytest.raises(p3.Pack3DError) as e:
        p3.build_index(c.to(DEV), (2, 2, 2), 1, ragged=True, offsets=[0, 4])
    assert e.value.status == p3.E_COORDS and "duplicate" in str(e.value) and "local index 2" in str(e.value)
    # tables sized for fewer blocks than the coordinates need
    lib = p3.load_library()
    cd = c[[0, 1, 3]].contiguous().to(DEV)
    pk = p3._packing(1, 3, ragged=True, max_blocks=1)
    bs = (p3.ctypes.c_int32 * 3)(2, 2, 2)
    nbytes = lib.pack3d_index_bytes(p3.ctypes.byref(pk), bs, 1)
    tables = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    h = p3.ctypes.c_void_p()
    st = lib.pack3d_build_index(p3._ptr(cd), p3.ctypes.byref(pk), bs, 1, p3._ptr(tables), nbytes,
                                p3.ctypes.c_void_p(p3._stream()), p3.ctypes.byref(h))
    assert st == p3.E_COORDS and b"needs 4 blocks" in lib.pack3d_last_error()


def test_autograd_wrapper_varlen():
    x = _inputs([(5, 6, 7), (4, 8, 5)], 2, 48, torch.float32, 0.7, seed=77)
    off = x["offsets"].tolist()
    xd = {k: v.to(DEV) for k, v in x.items() if k in ("q", "k", "v", "coords", "do")}
    ix = p3.build_index(xd["coords"], (2, 2, 2), 1, ragged=True, offsets=off)
    q, k, v = (xd[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = p3.attention(q, k, v, ix, xd["coords"])
    (o * xd["do"]).sum().backward()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], (2, 2, 2), 1, ragged=True,
                          offsets=np.asarray(off))
    for g, rr in zip((q.grad, k.grad, v.grad), ref):
        assert max_err(g, rr) < TOL[torch.float32]


def test_ragged_65k_scale_sampled():
    """The ragged stand-in at full size (about 111k tokens, two shapes): forward on sampled query
    blocks of both volumes, every gradient of one (volume, head)."""
    spec = si.RAGGED_WORKLOADS["65k-ragged"]
    dtype = torch.bfloat16
    say("ragged 65k-scale")
    x = _inputs(spec["grids"], spec["heads"], spec["head_dim"], dtype, spec["occupancy"], seed=spec["seed"])
    off = x["offsets"].numpy()
    _, out, lse, grads = _run(x, spec["block"], spec["radius"], dtype)
    blocks = [0, 5, 77, 500, 1000, 1500, 2000, 2500, 3000, 3550]
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], spec["block"], spec["radius"], ragged=True,
                                  offsets=off, query_blocks=blocks)
    mask = ~np.isnan(o_ref)
    assert mask.any()
    assert max_err(out, o_ref, mask) < TOL[dtype]
    assert max_err(lse, l_ref, ~np.isnan(l_ref)) < TOL[dtype]
    vol, head = 1, 3
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], spec["block"], spec["radius"], ragged=True,
                          offsets=off, volumes=[vol], heads=[head])
    a, b = off[vol], off[vol + 1]
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        gg = g[a:b, head].float().cpu().double().numpy()
        assert np.abs(gg - rr[a:b, head]).max() < TOL[dtype], name
        assert torch.isfinite(g).all(), name
