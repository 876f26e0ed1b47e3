"""Pins of the oracle's backward pass (gradients through RoPE and block pooling).

P10: central finite differences in fp64, and torch.autograd of an independent
dense-masked formulation on fp64 CPU (pooling as an explicit averaging matrix,
one softmax over a masked [keys | summaries] logit row).  Source of the
operator: "Geometry Matters in Packed 3D Attention", abstract ("trainable at
scale"); gradients are taken with respect to the unrotated q, k, v.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si


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
    """q, k, v [N, H, D] fp64 tensors; returns o [N, H, D]."""
    n, h, d = q.shape
    cc = c - c.min(0).values
    bc = cc // torch.tensor(block)
    keys, inv = torch.unique(bc, dim=0, return_inverse=True)        # blocks present
    pool = torch.zeros(keys.shape[0], n, dtype=torch.float64)
    pool[inv, torch.arange(n)] = 1.0
    pool = pool / pool.sum(1, keepdim=True)
    loc = (bc[:, None, :] - bc[None, :, :]).abs().amax(-1) <= r       # [N, N]
    far = (bc[:, None, :] - keys[None, :, :]).abs().amax(-1) > r      # [N, nblk]
    if not with_summaries:
        far = torch.zeros_like(far)
    qt, kt = _rope_torch(q, c, base), _rope_torch(k, c, base)
    kbar = torch.einsum("bn,nhd->bhd", pool, kt)
    vbar = torch.einsum("bn,nhd->bhd", pool, v)
    s = torch.einsum("ihd,jhd->hij", qt, kt) / math.sqrt(d)
    t = torch.einsum("ihd,bhd->hib", qt, kbar) / math.sqrt(d)
    s = s.masked_fill(~loc[None], float("-inf"))
    t = t.masked_fill(~far[None], float("-inf"))
    p = torch.softmax(torch.cat([s, t], -1), -1)
    vals = torch.cat([v.transpose(0, 1), vbar.transpose(0, 1)], 1)    # [H, N + nblk, D]
    return (p @ vals).transpose(0, 1)


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
