"""Pins of the oracle's forward pass ("Geometry Matters in Packed 3D Attention", abstract).

P1 repacking equivariance, P2 global-shift invariance, P3 rotate-before-pool
identity (a summary logit is the mean of the query's logits to the block's
rotated keys, a function of query-relative displacements only), P5-P7
reductions to dense 3D-RoPE attention (checked against torch's
scaled_dot_product_attention on fp64 CPU), P8 closed forms, P11 windowed-only
mode, and naive-versus-blocked agreement.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


def _inputs(w, **kw):
    x = si.make_inputs(w, torch.float32, **kw)
    return x["q"], x["k"], x["v"], x["coords"]


def _sdpa_reference(q, k, v, coords, base, mask=None):
    """Library dense attention (torch SDPA, fp64 CPU) on oracle-rotated q, k."""
    outs, lses = [], []
    for vi in range(q.shape[0]):
        qt = torch.from_numpy(oracle.rope(q[vi].double().numpy(), coords[vi].numpy(), base)).transpose(0, 1)
        kt = torch.from_numpy(oracle.rope(k[vi].double().numpy(), coords[vi].numpy(), base)).transpose(0, 1)
        vv = v[vi].double().transpose(0, 1)
        m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask[vi]))
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vv, attn_mask=m)
        s = qt @ kt.transpose(-1, -2) / math.sqrt(q.shape[-1])
        if m is not None:
            s = s.masked_fill(~m, float("-inf"))
        outs.append(o.transpose(0, 1).numpy())
        lses.append(torch.logsumexp(s, -1).numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("grid,block,r,with_s", [((4, 6, 8), (2, 2, 2), 1, True),
                                                 ((4, 4, 6), (2, 2, 3), 0, True),
                                                 ((6, 4, 4), (1, 2, 2), 1, False),
                                                 ((4, 4, 4), (2, 1, 2), 2, True)])
def test_naive_matches_blocked(grid, block, r, with_s):
    w = si.small_workload(grid=grid, block=block, radius=r, head_dim=12, heads=2, seed=5)
    q, k, v, c = _inputs(w)
    o1, l1 = oracle.forward(q, k, v, c, block, r, with_summaries=with_s)
    o2, l2 = oracle.forward_naive(q, k, v, c, block, r, with_summaries=with_s)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs(l1 - l2).max() < 1e-12


def test_repacking_equivariance_bitwise():
    """P1: the same physical tokens give bitwise-identical outputs under every packing."""
    w = si.small_workload(grid=(4, 6, 8), block=(2, 2, 2), head_dim=12, seed=9)
    ref = None
    for packing in si.PACKINGS:
        x = si.make_inputs(w, torch.float32, packing=packing)
        o, lse = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1)
        inv = np.argsort(x["perm"][0].numpy())          # raster index -> packed position
        o_r, l_r = o[0][inv], lse[0][:, inv]
        if ref is None:
            ref = (o_r, l_r)
        else:
            assert np.array_equal(o_r, ref[0]) and np.array_equal(l_r, ref[1]), packing


@pytest.mark.parametrize("shift", [(3, -5, 7), (-17, 1, 1), (1000, 0, -999)])
def test_global_shift_invariance(shift):
    """P2: shifting every coordinate by an integer vector leaves o and lse unchanged."""
    w = si.small_workload(grid=(4, 6, 8), block=(2, 3, 2), head_dim=24, seed=4)
    q, k, v, c = _inputs(w)
    q2, k2, v2, c2 = _inputs(w, shift=shift)
    o1, l1 = oracle.forward(q, k, v, c, w.block, 1)
    o2, l2 = oracle.forward(q2, k2, v2, c2, w.block, 1)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-11


def test_rotate_before_pool_logits():
    """P3: each logit equals scale * q_i^T R(c_j - c_i) k_j (mean over the block for summaries)."""
    w = si.small_workload(grid=(4, 4, 6), block=(2, 2, 2), head_dim=12, heads=2, seed=13)
    q, k, v, c = _inputs(w)
    o, lse, lg_loc, lg_sum = oracle.forward(q, k, v, c, w.block, 1, return_logits=True)
    qn, kn, cn = q[0].double().numpy(), k[0].double().numpy(), c[0].numpy().astype(np.int64)
    n, h, d = qn.shape
    scale = 1 / math.sqrt(d)
    bc = (cn - cn.min(0)) // np.array(w.block)
    blocks = sorted({tuple(x) for x in bc.tolist()})
    nb = np.array(w.grid) // np.array(w.block)
    rng = np.random.default_rng(0)
    for i in rng.choice(n, 12, replace=False):
        rel = oracle.rope(kn, cn - cn[i])                  # R(c_j - c_i) k_j, every j
        direct = scale * (rel * qn[i][None]).sum(-1)       # [N, H]
        for j in range(n):
            if np.abs(bc[j] - bc[i]).max() <= 1:
                assert abs(lg_loc[0, :, i, j] - direct[j]).max() < 1e-12
            else:
                assert np.isnan(lg_loc[0, :, i, j]).all()
        for blk in blocks:
            bid = (blk[0] * nb[1] + blk[1]) * nb[2] + blk[2]
            members = (bc == np.array(blk)).all(1)
            if max(abs(a - b) for a, b in zip(blk, bc[i])) > 1:
                assert abs(lg_sum[0, :, i, bid] - direct[members].mean(0)).max() < 1e-12
            else:
                assert np.isnan(lg_sum[0, :, i, bid]).all()


@pytest.mark.parametrize("grid,block,r", [((8, 8, 8), (2, 2, 2), 3), ((4, 6, 8), (2, 2, 2), 3)])
def test_dense_reduction_large_radius(grid, block, r):
    """P5 (and P11): a radius covering the block grid gives dense 3D-RoPE attention."""
    w = si.small_workload(grid=grid, block=block, head_dim=12, heads=2, seed=21)
    q, k, v, c = _inputs(w)
    od, ld = _sdpa_reference(q, k, v, c, w.rope_base)
    for with_s in (True, False):
        o, lse = oracle.forward(q, k, v, c, block, r, with_summaries=with_s)
        assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def test_dense_reduction_unit_blocks():
    """P6: 1x1x1 blocks make every summary one rotated key -> dense attention at any radius."""
    w = si.small_workload(grid=(4, 4, 6), block=(1, 1, 1), head_dim=18, heads=2, seed=22)
    q, k, v, c = _inputs(w)
    od, ld = _sdpa_reference(q, k, v, c, w.rope_base)
    for r in (0, 1):
        o, lse = oracle.forward(q, k, v, c, (1, 1, 1), r)
        assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def test_dense_reduction_single_block():
    """P7: one block spanning the grid -> dense attention."""
    w = si.small_workload(grid=(4, 4, 6), block=(4, 4, 6), head_dim=12, seed=23)
    q, k, v, c = _inputs(w)
    od, ld = _sdpa_reference(q, k, v, c, w.rope_base)
    o, lse = oracle.forward(q, k, v, c, w.block, 0)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def test_windowed_only_is_masked_dense():
    """Windowed-only mode = softmax over the local keys only (brute-force Chebyshev mask)."""
    w = si.small_workload(grid=(4, 6, 8), block=(2, 2, 2), head_dim=12, seed=24)
    q, k, v, c = _inputs(w)
    cn = c[0].numpy()
    bc = (cn - cn.min(0)) // np.array(w.block)
    mask = (np.abs(bc[:, None, :] - bc[None, :, :]).max(-1) <= 1)[None, None]
    od, ld = _sdpa_reference(q, k, v, c, w.rope_base, mask=np.broadcast_to(mask, (1, 2) + mask.shape[2:]))
    o, lse = oracle.forward(q, k, v, c, w.block, 1, with_summaries=False)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def test_closed_forms():
    """P8: constant V gives constant o; q = 0 gives the plain mean of local values and summaries."""
    w = si.small_workload(grid=(4, 6, 8), block=(2, 2, 2), head_dim=12, seed=25)
    q, k, v, c = _inputs(w)
    vc = torch.full_like(v, 0.375)
    o, _ = oracle.forward(q, k, vc, c, w.block, 1)
    assert np.abs(o - 0.375).max() < 1e-13
    q0 = torch.zeros_like(q)
    o, lse = oracle.forward(q0, k, v, c, w.block, 1)
    cn = c[0].numpy()
    vn = v[0].double().numpy()
    bc = (cn - cn.min(0)) // np.array(w.block)
    keys = {tuple(x) for x in bc.tolist()}
    for i in range(0, cn.shape[0], 7):
        loc = np.abs(bc - bc[i]).max(1) <= 1
        far = [b for b in keys if max(abs(a - bb) for a, bb in zip(b, bc[i])) > 1]
        means = [vn[(bc == np.array(b)).all(1)].mean(0) for b in far]
        total = vn[loc].sum(0) + sum(means)
        cnt = loc.sum() + len(far)
        assert np.abs(o[0, i] - total / cnt).max() < 1e-13
        assert np.abs(lse[0, :, i] - math.log(cnt)).max() < 1e-13


def test_query_block_sampling_matches_full():
    w = si.small_workload(grid=(4, 6, 8), block=(2, 2, 2), head_dim=12, seed=26, batch=2)
    q, k, v, c = _inputs(w)
    o, lse = oracle.forward(q, k, v, c, w.block, 1)
    os_, ls = oracle.forward(q, k, v, c, w.block, 1, query_blocks=[0, 5, 11])
    ok = ~np.isnan(os_)
    assert ok.sum() == 2 * 3 * 8 * 2 * 12
    assert np.array_equal(os_[ok], o[ok])
    assert np.array_equal(ls[~np.isnan(ls)], lse[~np.isnan(ls)])


def test_dense_attention_matches_library():
    """oracle.dense_attention (plain softmax attention with 3D RoPE) against torch SDPA on fp64 CPU."""
    w = si.small_workload(grid=(4, 4, 6), block=(2, 2, 2), head_dim=12, heads=2, seed=27, batch=2)
    q, k, v, c = _inputs(w)
    od, ld = _sdpa_reference(q, k, v, c, w.rope_base)
    o, lse = oracle.dense_attention(q, k, v, c, rope_base=w.rope_base)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12
