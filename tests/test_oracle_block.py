"""Pins of the oracle transformer block around PACK3D (oracle/block.py).

The block is a reading (the pages give no layer layout): pre-norm, one fused QKV
projection, the operator, an output projection, and a GELU MLP, each with a residual.
Pins: with a radius covering the block grid the operator is dense 3D-RoPE attention, so the
block must equal the same block built on torch SDPA (fp64) with an independent complex-
number RoPE, forward and every gradient; central finite differences of a block whose
operator has distant summaries pin the oracle operator's gradients inside the block; planted
mistakes in the block wiring fail the dense pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle.block as ob
import synthetic_inputs as si
from tests.dense_ref import torch_axial_rope


def _sdpa_attention(coords):
    c = torch.from_numpy(np.asarray(coords)).long()

    def att(q, k, v):   # q, k, v [1, N, H, D]
        qt = torch_axial_rope(q[0], c).transpose(0, 1)
        kt = torch_axial_rope(k[0], c).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, v[0].transpose(0, 1))
        return o.transpose(0, 1)[None]
    return att


def _setup(grid, block, heads, d, seed):
    w = si.small_workload(grid=grid, block=block, heads=heads, head_dim=d, packing="random", seed=seed)
    coords = si.make_inputs(w, torch.float32)["coords"].numpy()
    n = int(np.prod(grid))
    g = np.random.default_rng(seed + 1)
    x = torch.from_numpy(g.standard_normal((1, n, heads * d)))
    dy = torch.from_numpy(g.standard_normal((1, n, heads * d)))
    return coords, x, dy, ob.init_params(heads * d, seed=seed)


def _grads(x, params, dy, **kw):
    x = x.clone().requires_grad_()
    ps = {k: v.clone().requires_grad_() for k, v in params.items()}
    y = ob.block_forward(x, ps, **kw)
    (y * dy).sum().backward()
    return y.detach(), x.grad, {k: v.grad for k, v in ps.items()}


def test_dense_reduction_against_sdpa_block():
    coords, x, dy, params = _setup((4, 4, 4), (2, 2, 2), 2, 12, seed=81)
    kw = dict(coords=coords, block_shape=(2, 2, 2), radius=2, heads=2)
    y, gx, gp = _grads(x, params, dy, **kw)
    y2, gx2, gp2 = _grads(x, params, dy, attention=_sdpa_attention(coords[0]), **kw)
    np.testing.assert_allclose(y, y2, atol=1e-12)
    np.testing.assert_allclose(gx, gx2, atol=1e-10)
    for k in params:
        np.testing.assert_allclose(gp[k], gp2[k], atol=1e-10, err_msg=k)


def test_finite_differences_with_summaries():
    coords, x, dy, params = _setup((4, 4, 6), (2, 2, 2), 2, 6, seed=82)
    kw = dict(coords=coords, block_shape=(2, 2, 2), radius=1, heads=2)
    _, gx, gp = _grads(x, params, dy, **kw)

    def loss(xx, pp):
        return float((ob.block_forward(xx, pp, **kw) * dy).sum())

    h = 1e-6
    rng = np.random.default_rng(3)
    for _ in range(6):
        i, j = int(rng.integers(0, x.shape[1])), int(rng.integers(0, x.shape[2]))
        xp, xm = x.clone(), x.clone()
        xp[0, i, j] += h
        xm[0, i, j] -= h
        fd = (loss(xp, params) - loss(xm, params)) / (2 * h)
        assert abs(fd - float(gx[0, i, j])) < 1e-6 * max(1.0, abs(fd)), (i, j, fd, float(gx[0, i, j]))
    for name in ("qkv", "proj", "fc1", "ln2_w"):
        p = params[name]
        idx = tuple(int(rng.integers(0, s)) for s in p.shape)
        pp, pm = dict(params), dict(params)
        pp[name], pm[name] = p.clone(), p.clone()
        pp[name][idx] += h
        pm[name][idx] -= h
        fd = (loss(x, pp) - loss(x, pm)) / (2 * h)
        assert abs(fd - float(gp[name][idx])) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, float(gp[name][idx]))


@pytest.mark.parametrize("mistake", ["swap_qk", "proj_transposed"])
def test_planted_wiring_mistakes_fail_dense_pin(monkeypatch, mistake):
    coords, x, dy, params = _setup((4, 4, 4), (2, 2, 2), 2, 12, seed=83)
    kw = dict(coords=coords, block_shape=(2, 2, 2), radius=2, heads=2)
    y_ref = ob.block_forward(x, params, attention=_sdpa_attention(coords[0]), **kw)
    bad = dict(params)
    if mistake == "swap_qk":
        c = x.shape[-1]
        w = params["qkv"].clone()
        bad["qkv"] = torch.cat([w[c:2 * c], w[:c], w[2 * c:]])
    else:
        bad["proj"] = params["proj"].T.clone()
    y = ob.block_forward(x, bad, **kw)
    assert float((y - y_ref).abs().max()) > 1e-3
