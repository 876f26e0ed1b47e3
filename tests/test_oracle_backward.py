"""Pins of the oracle's backward pass (gradients through RoPE and block pooling).

P10: central finite differences in fp64, and torch.autograd of an independent
dense-masked formulation on fp64 CPU (pooling as an explicit averaging matrix,
one softmax over a masked [keys | summaries] logit row).  Source of the
operator: "Geometry Matters in Packed 3D Attention", abstract ("trainable at
scale"); gradients are taken with respect to the unrotated q, k, v.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tests.dense_ref import dense_masked


def _rope_torch(x, c, base):
    d = x.shape[-1]
    da, half = d // 3, d // 6
    theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / da)
    parts = []
    for a in range(3):
        phi = c[:, a:a + 1].double() * theta[None]          # [N, half]
        cos, sin = torch.cos(phi)[:, None], torch.sin(phi)[:, None]
        x1 = x[..., a * da:a * da + half]
        x2 = x[..., a * da + half:(a + 1) * da]
        parts += [x1 * cos - x2 * sin, x1 * sin + x2 * cos]
    return torch.cat(parts, -1)


def _dense_masked(q, k, v, c, block, r, base, with_summaries=True):
    """q, k, v [N, H, D] fp64 tensors; returns o [N, H, D] of the dense-masked formulation
    (``tests/dense_ref.py``) with the real cos / sin rotation above."""
    return dense_masked(q, k, v, c, block, r, lambda x: _rope_torch(x, c, base), with_summaries)


@pytest.mark.parametrize("grid,block,r,with_s", [((4, 4, 6), (2, 2, 2), 1, True),
                                                 ((4, 6, 4), (1, 2, 2), 1, True),
                                                 ((4, 4, 4), (2, 2, 2), 0, False),
                                                 ((6, 4, 4), (2, 2, 1), 2, True)])
def test_backward_matches_autograd_of_dense_masked_formulation(grid, block, r, with_s):
    w = si.small_workload(grid=grid, block=block, head_dim=12, heads=2, seed=31, batch=2)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], block, r,
                                 with_summaries=with_s)
    o_or, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], block, r, with_summaries=with_s)
    for vi in range(2):
        q = x["q"][vi].double().requires_grad_()
        k = x["k"][vi].double().requires_grad_()
        v = x["v"][vi].double().requires_grad_()
        o = _dense_masked(q, k, v, x["coords"][vi].long(), block, r, w.rope_base, with_s)
        assert (o.detach().numpy() - o_or[vi]).__abs__().max() < 1e-12
        (o * x["do"][vi].double()).sum().backward()
        for got, ref in ((dq[vi], q.grad), (dk[vi], k.grad), (dv[vi], v.grad)):
            assert np.abs(got - ref.numpy()).max() < 1e-12


def test_backward_central_differences():
    w = si.small_workload(grid=(2, 4, 4), block=(1, 2, 2), head_dim=6, heads=1, seed=32)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    c, do = x["coords"], x["do"].double().numpy()
    dq, dk, dv = oracle.backward(q, k, v, c, do, w.block, 1)
    h = 1e-6
    rng = np.random.default_rng(1)

    def f(qq, kk, vv):
        return (oracle.forward(qq, kk, vv, c, w.block, 1)[0] * do).sum()

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(3):
            e = rng.standard_normal(q.shape)
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which] += h * e
            args_m[which] -= h * e
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            assert abs(fd - (grad * e).sum()) < 1e-7 * max(1.0, abs(fd))


def test_backward_sampling_by_volume_and_head():
    w = si.small_workload(grid=(4, 4, 4), block=(2, 2, 2), head_dim=12, heads=3, seed=33, batch=2)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    full = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    part = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1, volumes=[1], heads=[2])
    for a, b in zip(full, part):
        assert np.array_equal(a[1][:, 2], b[1][:, 2])
        assert np.isnan(b[0]).all() and np.isnan(b[1][:, :2]).all()


def test_backward_repacking_equivariance_bitwise():
    w = si.small_workload(grid=(4, 4, 6), block=(2, 2, 2), head_dim=12, seed=34)
    ref = None
    for packing in si.PACKINGS:
        x = si.make_inputs(w, torch.float32, packing=packing, with_grad=True)
        g = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
        inv = np.argsort(x["perm"][0].numpy())
        g = [t[0][inv] for t in g]
        if ref is None:
            ref = g
        else:
            for a, b in zip(g, ref):
                assert np.array_equal(a, b), packing


def test_backward_query_block_sampling_matches_full():
    """dq of sampled query blocks equals the full pass bitwise; dk and dv are not returned."""
    w = si.small_workload(grid=(4, 4, 6), block=(2, 2, 2), head_dim=12, heads=2, seed=35, batch=2)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    full = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    part = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1, query_blocks=[0, 4, 11])
    ok = ~np.isnan(part[0])
    assert ok.sum() == 2 * 3 * 8 * 2 * 12
    assert np.array_equal(part[0][ok], full[0][ok])
    assert np.isnan(part[1]).all() and np.isnan(part[2]).all()
    y = si.make_ragged_inputs([(5, 4, 6), (3, 6, 4)], 2, 12, occupancy=0.7, seed=36, with_grad=True)
    off = y["offsets"].numpy()
    full = oracle.backward(y["q"], y["k"], y["v"], y["coords"], y["do"], (2, 2, 2), 1, ragged=True, offsets=off)
    part = oracle.backward(y["q"], y["k"], y["v"], y["coords"], y["do"], (2, 2, 2), 1, ragged=True, offsets=off,
                           query_blocks=[1, 7])
    ok = ~np.isnan(part[0])
    assert 0 < ok.sum() < ok.size
    assert np.array_equal(part[0][ok], full[0][ok])


def _conservation(q, k, v, c, do, block, r, with_s=True, offsets=None, ragged=False):
    """(sum_j dv_j - sum_i do_i, sum_j R_j dk_j) per volume, fp64 [H, D] each."""
    dq, dk, dv = oracle.backward(q, k, v, c, do, block, r, with_summaries=with_s, offsets=offsets, ragged=ragged)
    res = []
    if offsets is None:
        vols = [(dk[b], dv[b], do[b].double(), c[b]) for b in range(q.shape[0])]
    else:
        vols = [(dk[a:e], dv[a:e], do[a:e].double(), c[a:e]) for a, e in zip(offsets[:-1], offsets[1:])]
    for dkv, dvv, dov, cv in vols:
        rel = torch.as_tensor(cv).long()
        rel = rel - rel.min(0).values
        rot = _rope_torch(torch.from_numpy(dkv), rel, 10000.0)
        res.append((dvv.sum(0) - dov.numpy().sum(0), rot.sum(0).numpy()))
    return res


@pytest.mark.parametrize("grid,block,r,with_s", [((4, 6, 8), (2, 2, 2), 1, True),
                                                 ((4, 6, 8), (2, 2, 2), 1, False),
                                                 ((4, 4, 8), (2, 2, 4), 0, True)])
def test_backward_conservation_laws(grid, block, r, with_s):
    """Each query's softmax weights sum to one, so (i) the value gradients add up to the sum of
    dO over queries, and (ii) the rotated key gradients R_j dk_j add up to zero (every score row
    has zero-sum dS); block means hand each summary's gradient to its members in full."""
    w = si.small_workload(grid=grid, block=block, head_dim=12, heads=2, seed=37, batch=2)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    do = x["do"] + 0.75                 # a mean offset makes the value-gradient sum large
    for dv_gap, dk_sum in _conservation(x["q"], x["k"], x["v"], x["coords"], do, block, r, with_s):
        assert np.abs(dv_gap).max() < 1e-11
        assert np.abs(dk_sum).max() < 1e-11


def test_backward_conservation_laws_ragged():
    y = si.make_ragged_inputs([(5, 4, 6), (3, 6, 4)], 2, 12, occupancy=0.6, seed=38, with_grad=True)
    off = y["offsets"].numpy()
    do = y["do"] + 0.75
    for dv_gap, dk_sum in _conservation(y["q"], y["k"], y["v"], y["coords"], do, (2, 2, 2), 1,
                                        offsets=off, ragged=True):
        assert np.abs(dv_gap).max() < 1e-11
        assert np.abs(dk_sum).max() < 1e-11
