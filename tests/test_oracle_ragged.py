"""Pins of the oracle's ragged geometry and varlen batches.

"Geometry Matters in Packed 3D Attention" (abstract): the operator serves packed
geometric data in general.  With ``ragged=True`` a volume is any set of distinct
integer points: extents that the block does not divide (partial edge blocks) and holes
(sparse occupancy).  Blocks cover the bounding box from its minimum corner; the local
set is the present tokens of the blocks within the radius; every other occupied block
gives one summary, the mean over the tokens present in it; an empty block gives none.
A batch of volumes with different token counts is flat with ``offsets``.

Pins: the token-by-token definition (no tables), reductions to dense attention
(torch SDPA) by radius and by unit blocks, closed forms that count local keys and
occupied summaries, repacking and shift behaviour, batch independence of a varlen
batch, identity with the full-grid path on full grids, and autograd of an independent
dense-masked formulation for the gradients.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tests.dense_ref import dense_masked, torch_axial_rope

CASES = [
    # grids (one per volume), block, radius, occupancy
    ([(5, 6, 7)], (2, 2, 2), 1, 0.7),
    ([(4, 5, 9), (6, 3, 5)], (2, 2, 3), 1, 0.8),
    ([(7, 4, 4)], (3, 2, 2), 0, 0.6),
    ([(6, 6, 6), (3, 7, 4)], (2, 2, 2), 2, 0.5),
]


def _np(t):
    return t.double().numpy()


def _volume(x, v):
    """Volume v of a flat ragged batch as a one-volume [1, N, ...] batch."""
    a, b = int(x["offsets"][v]), int(x["offsets"][v + 1])
    return {k: x[k][a:b][None] for k in ("q", "k", "v", "coords", "do") if k in x}


@pytest.mark.parametrize("grids,block,r,occ", CASES)
@pytest.mark.parametrize("mode", ["axial", "none"])
def test_ragged_matches_token_by_token_definition(grids, block, r, occ, mode):
    x = si.make_ragged_inputs(grids, 2, 12, occupancy=occ, seed=51)
    for v in range(len(grids)):
        y = _volume(x, v)
        for with_s in (True, False):
            o, lse = oracle.forward(y["q"], y["k"], y["v"], y["coords"], block, r, ragged=True,
                                    with_summaries=with_s, position_mode=mode)
            o2, lse2 = oracle.forward_naive(y["q"], y["k"], y["v"], y["coords"], block, r,
                                            with_summaries=with_s, position_mode=mode)
            np.testing.assert_allclose(o, o2, atol=1e-12)
            np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_varlen_batch_equals_separate_volumes():
    """Volumes never interact: the flat call equals one call per volume, bitwise; lse is
    [B, H, max N_v] with NaN past each volume's tokens."""
    grids = [(5, 6, 7), (4, 4, 9), (6, 3, 5)]
    x = si.make_ragged_inputs(grids, 2, 12, occupancy=0.75, seed=52, with_grad=True)
    off = x["offsets"].numpy()
    o, lse = oracle.forward(x["q"], x["k"], x["v"], x["coords"], (2, 2, 2), 1, ragged=True, offsets=off)
    grads = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], (2, 2, 2), 1, ragged=True, offsets=off)
    nmax = int(np.diff(off).max())
    assert o.shape == tuple(x["q"].shape) and lse.shape == (3, 2, nmax)
    for v in range(3):
        y = _volume(x, v)
        n = off[v + 1] - off[v]
        o1, l1 = oracle.forward(y["q"], y["k"], y["v"], y["coords"], (2, 2, 2), 1, ragged=True)
        np.testing.assert_array_equal(o[off[v]:off[v + 1]], o1[0])
        np.testing.assert_array_equal(lse[v, :, :n], l1[0])
        assert np.isnan(lse[v, :, n:]).all()
        g1 = oracle.backward(y["q"], y["k"], y["v"], y["coords"], y["do"], (2, 2, 2), 1, ragged=True)
        for g, ref in zip(grads, g1):
            np.testing.assert_array_equal(g[off[v]:off[v + 1]], ref[0])


def test_full_grid_same_as_full_path():
    """On a full grid divisible by the block the ragged path is the full-grid path, bitwise."""
    w = si.small_workload(grid=(4, 6, 8), block=(2, 2, 2), heads=2, head_dim=12, packing="random", seed=53)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    a = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1)
    b = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1, ragged=True)
    for u, t in zip(a, b):
        np.testing.assert_array_equal(u, t)
    ga = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    gb = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1, ragged=True)
    for u, t in zip(ga, gb):
        np.testing.assert_array_equal(u, t)


def _sdpa(q, k, v, c, base=10000.0):
    """Dense attention over the present tokens: torch SDPA (fp64 CPU) on axial-rotated q, k."""
    qt = torch.from_numpy(oracle.rope(_np(q), c.numpy(), base)).transpose(0, 1)
    kt = torch.from_numpy(oracle.rope(_np(k), c.numpy(), base)).transpose(0, 1)
    vv = v.double().transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vv)
    lse = torch.logsumexp(qt @ kt.transpose(-1, -2) / math.sqrt(q.shape[-1]), -1)
    return o.transpose(0, 1).numpy(), lse.numpy()


def test_dense_reduction_large_radius():
    """A radius covering the block grid: every present token is local, no summaries."""
    x = si.make_ragged_inputs([(5, 6, 7)], 2, 12, occupancy=0.6, seed=54)
    o, lse = oracle.forward(x["q"][None], x["k"][None], x["v"][None], x["coords"][None], (2, 2, 3), 3,
                            ragged=True)
    od, ld = _sdpa(x["q"], x["k"], x["v"], x["coords"])
    np.testing.assert_allclose(o[0], od, atol=1e-12)
    np.testing.assert_allclose(lse[0], ld, atol=1e-12)


@pytest.mark.parametrize("r", [0, 1, 2])
def test_dense_reduction_unit_blocks(r):
    """1x1x1 blocks: each summary is one rotated key and its value, so any radius gives dense
    attention over the present tokens."""
    x = si.make_ragged_inputs([(4, 5, 6)], 2, 12, occupancy=0.55, seed=55)
    o, lse = oracle.forward(x["q"][None], x["k"][None], x["v"][None], x["coords"][None], (1, 1, 1), r,
                            ragged=True)
    od, ld = _sdpa(x["q"], x["k"], x["v"], x["coords"])
    np.testing.assert_allclose(o[0], od, atol=1e-12)
    np.testing.assert_allclose(lse[0], ld, atol=1e-12)


def test_closed_form_counts_present_keys_and_occupied_blocks():
    """q = 0: every logit is 0, so o_i = (sum of local v + sum of summaries) / (|L(i)| + |S(i)|)
    and lse_i = ln(|L(i)| + |S(i)|), where |L(i)| counts the present tokens of the local blocks
    and |S(i)| the occupied non-local blocks.  A whole block is emptied so that it must give no
    summary, and the edge blocks are partial."""
    grid, block, r = (6, 5, 9), (2, 2, 3), 1
    x = si.make_ragged_inputs([grid], 2, 12, occupancy=0.7, seed=56)
    c = x["coords"].numpy().astype(np.int64)
    keep = ~(((c[:, 0] // 2) == 1) & ((c[:, 1] // 2) == 2) & ((c[:, 2] // 3) == 1))   # empty block (1, 2, 1)
    q = torch.zeros_like(x["q"][keep])
    k, v, cc = x["k"][keep], x["v"][keep], x["coords"][keep]
    o, lse = oracle.forward(q[None], k[None], v[None], cc[None], block, r, ragged=True)
    c = cc.numpy().astype(np.int64)
    bc = (c - c.min(0)) // np.asarray(block)
    vv = _np(v)
    blocks = {tuple(b) for b in bc.tolist()}
    assert (1, 2, 1) not in blocks
    vbar = {b: vv[(bc == np.asarray(b)).all(1)].mean(0) for b in blocks}
    for i in range(c.shape[0]):
        loc = np.abs(bc - bc[i]).max(1) <= r
        far = [b for b in blocks if max(abs(p - s) for p, s in zip(b, bc[i])) > r]
        cnt = loc.sum() + len(far)
        want = (vv[loc].sum(0) + sum(vbar[b] for b in far)) / cnt
        np.testing.assert_allclose(o[0, i], want, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, i], math.log(cnt), atol=1e-12)


def test_repacking_bitwise_and_shift_invariance():
    x = si.make_ragged_inputs([(5, 7, 6)], 2, 12, occupancy=0.65, seed=57, with_grad=True)
    args = dict(block_shape=(2, 2, 2), local_radius=1, ragged=True)
    o, lse = oracle.forward(x["q"][None], x["k"][None], x["v"][None], x["coords"][None], **args)
    g = oracle.backward(x["q"][None], x["k"][None], x["v"][None], x["coords"][None], x["do"][None], **args)
    p = torch.from_numpy(np.random.default_rng(9).permutation(x["q"].shape[0]))
    y = {k: x[k][p] for k in ("q", "k", "v", "coords", "do")}
    o2, lse2 = oracle.forward(y["q"][None], y["k"][None], y["v"][None], y["coords"][None], **args)
    g2 = oracle.backward(y["q"][None], y["k"][None], y["v"][None], y["coords"][None], y["do"][None], **args)
    pn = p.numpy()
    np.testing.assert_array_equal(o2[0], o[0][pn])
    np.testing.assert_array_equal(lse2[0], lse[0][:, pn])
    for a, b in zip(g2, g):
        np.testing.assert_array_equal(a[0], b[0][pn])
    # a shift that is not a multiple of the block moves the lattice with the data
    sc = x["coords"] + torch.tensor([-3, 5, 1], dtype=torch.int32)
    o3, lse3 = oracle.forward(x["q"][None], x["k"][None], x["v"][None], sc[None], **args)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(lse3, lse, atol=1e-12)


@pytest.mark.parametrize("mode", ["axial", "none"])
def test_backward_against_autograd(mode):
    x = si.make_ragged_inputs([(5, 4, 7), (3, 6, 5)], 2, 12, occupancy=0.7, seed=58, with_grad=True)
    off = x["offsets"].numpy()
    grads = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], (2, 2, 3), 1, ragged=True, offsets=off,
                            position_mode=mode)
    for v in range(2):
        y = _volume(x, v)
        c = y["coords"][0].long()
        if mode == "axial":
            rot = lambda t, c=c: torch_axial_rope(t, c)       # noqa: E731
        else:
            rot = lambda t: t                                    # noqa: E731
        q, k, vv = (y[n][0].double().clone().requires_grad_() for n in ("q", "k", "v"))
        o = dense_masked(q, k, vv, c, (2, 2, 3), 1, rot)
        (o * y["do"][0].double()).sum().backward()
        for g, ref in zip(grads, (q.grad, k.grad, vv.grad)):
            np.testing.assert_allclose(g[off[v]:off[v + 1]], ref.numpy(), atol=1e-11)


def test_geometry_errors():
    c = np.array([[0, 0, 0], [0, 0, 1], [0, 1, 0]])
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(c, (1, 1, 1), 1)
    assert e.value.reason == "grid"
    ix = oracle.build_index(c, (1, 2, 2), 1, ragged=True)[0]
    assert ix["nblk"] == 1 and ix["count"].tolist() == [3] and (ix["perm"] >= 0).sum() == 3
    with pytest.raises(oracle.CoordsError) as e:
        oracle.build_index(np.array([[0, 0, 0], [1, 1, 1], [0, 0, 0]]), (1, 1, 1), 1, ragged=True)
    assert e.value.reason == "duplicate" and e.value.token == 2


def test_ragged_tables_closed_forms():
    """nb = ceil(extent / b); block counts sum to N; perm inverts canon; empty slots are -1."""
    x = si.make_ragged_inputs([(7, 5, 9)], 1, 6, occupancy=0.5, seed=59)
    c = x["coords"].numpy()
    ix = oracle.build_index(c, (2, 2, 4), 1, ragged=True)[0]
    assert ix["nb"].tolist() == [4, 3, 3]
    assert ix["count"].sum() == c.shape[0]
    np.testing.assert_array_equal(ix["perm"][ix["canon"]], np.arange(c.shape[0]))
    assert (ix["perm"] >= 0).sum() == c.shape[0]
    # each block's count equals a brute-force count of the points inside its box
    rel = c - c.min(0)
    for bid in range(ix["nblk"]):
        bz, rem = divmod(bid, 9)
        by, bx = divmod(rem, 3)
        inside = ((rel[:, 0] // 2 == bz) & (rel[:, 1] // 2 == by) & (rel[:, 2] // 4 == bx)).sum()
        assert ix["count"][bid] == inside
