"""Pins of the oracle's position modes (controls of the operator).

"Geometry Matters in Packed 3D Attention" (abstract): position encodings indexed by the
packed sequence learn the memory layout and collapse under repacking, while axial RoPE
on grid coordinates does not.  The oracle's ``position_mode`` keeps the operator's
locality and summaries and swaps only the rotation: "axial" (the method), "packed1d"
(standard RoPE on the packed position, the 1D rotation of the "SpatioTemporal RoPE"
section over the whole head dim) and "none".

Pins: closed forms of the 1D rotation, its group properties, an independent complex
formulation, reductions to dense attention against torch SDPA, the token-by-token
definition, the repacking behaviour the pages describe, and torch.autograd of an
independent dense-masked formulation for the gradients.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.pack3d as op
import synthetic_inputs as si
from tests.dense_ref import dense_masked


def _complex_rope_1d(x, pos, base):
    """1D RoPE through complex multiplication: pair (k, k + D/2) is the complex number
    x_k + i x_{k+D/2}, turned by exp(i * pos * base^(-2k/D))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = np.exp(np.log(base) * (-np.arange(d // 2) * 2.0 / d))
    w = np.exp(1j * np.multiply.outer(np.asarray(pos, dtype=np.float64), freq))   # [N, D/2]
    if x.ndim == 3:
        w = w[:, None, :]
    zr = z * w
    return np.concatenate([zr.real, zr.imag], axis=-1)


def test_rope_1d_closed_forms():
    # D = 2: one pair with theta_0 = 1, position 1 turns by one radian
    x = np.array([[0.3, -1.7]])
    c, s = math.cos(1.0), math.sin(1.0)
    want = np.array([[0.3 * c + 1.7 * s, 0.3 * s - 1.7 * c]])
    np.testing.assert_allclose(op.rope_1d(x, np.array([1]), 10000.0), want, rtol=0, atol=1e-15)
    # D = 4, base 1e4: theta_1 = 1e4^(-1/2) = 0.01, so position 100 turns pair (1, 3) by one radian
    x = np.zeros((1, 4))
    x[0, 1] = 1.0
    out = op.rope_1d(x, np.array([100]), 10000.0)
    np.testing.assert_allclose(out, [[0.0, c, 0.0, s]], rtol=0, atol=1e-14)
    # pair (0, 2) at the same position turns by 100 radians (theta_0 = 1)
    x = np.zeros((1, 4))
    x[0, 0] = 1.0
    out = op.rope_1d(x, np.array([100]), 10000.0)
    np.testing.assert_allclose(out, [[math.cos(100.0), 0.0, math.sin(100.0), 0.0]], rtol=0, atol=1e-13)


def test_rope_1d_group_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 3, 12))
    y = rng.standard_normal((40, 3, 12))
    pos_a = rng.integers(0, 5000, 40)
    pos_b = rng.integers(0, 5000, 40)
    np.testing.assert_array_equal(op.rope_1d(x, np.zeros(40, dtype=int)), x)
    np.testing.assert_allclose(op.rope_1d(op.rope_1d(x, pos_a), pos_a, inverse=True), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(op.rope_1d(x, pos_a), axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-12)
    # <R(a) x, R(b) y> = <x, R(b - a) y>: logits depend on the position difference only
    lhs = (op.rope_1d(x, pos_a) * op.rope_1d(y, pos_b)).sum(-1)
    rhs = (x * op.rope_1d(y, pos_b - pos_a)).sum(-1)
    np.testing.assert_allclose(lhs, rhs, atol=1e-10)


def test_rope_1d_matches_complex_formulation():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 2, 48))
    pos = rng.permutation(64)
    np.testing.assert_allclose(op.rope_1d(x, pos, 500.0), _complex_rope_1d(x, pos, 500.0), atol=1e-12)


def test_planted_adjacent_pairing_is_caught():
    """Negative control: an interleaved-pair 1D RoPE ((2k, 2k+1) pairs) fails the complex pin."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 8))
    pos = np.arange(16)
    theta = op.rope_tables(8, 10000.0)
    phi = pos[:, None] * theta[None]
    wrong = np.empty_like(x)
    wrong[:, 0::2] = x[:, 0::2] * np.cos(phi) - x[:, 1::2] * np.sin(phi)
    wrong[:, 1::2] = x[:, 0::2] * np.sin(phi) + x[:, 1::2] * np.cos(phi)
    assert np.abs(wrong - _complex_rope_1d(x, pos, 10000.0)).max() > 1e-2


def _sdpa(q, k, v):
    """Dense attention via torch SDPA on fp64 CPU; q, k, v [N, H, D] numpy."""
    t = [torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*t)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("mode", ["none", "packed1d"])
def test_dense_reduction_against_sdpa(mode):
    """Radius covering the grid: every key is local, no summaries; equals dense attention with
    the mode's rotation applied at the packed positions."""
    w = si.small_workload(grid=(4, 4, 4), block=(2, 2, 2), radius=2, heads=2, head_dim=12, packing="random",
                          seed=31)
    x = si.make_inputs(w, torch.float32)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 2, position_mode=mode)
    q, k, v = (x[n][0].double().numpy() for n in ("q", "k", "v"))
    if mode == "packed1d":
        pos = np.arange(q.shape[0])                          # packed order: index = position
        q, k = _complex_rope_1d(q, pos, 10000.0), _complex_rope_1d(k, pos, 10000.0)
    np.testing.assert_allclose(o[0], _sdpa(q, k, v), atol=1e-12)


@pytest.mark.parametrize("mode", ["none", "packed1d"])
def test_blocked_matches_token_by_token_definition(mode):
    w = si.small_workload(grid=(4, 4, 8), block=(2, 2, 2), radius=1, heads=2, head_dim=12, packing="morton",
                          seed=32)
    x = si.make_inputs(w, torch.float32)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1, position_mode=mode)
    o2, lse2 = oracle.forward_naive(x["q"], x["k"], x["v"], x["coords"], w.block, 1, position_mode=mode)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_repacking_axial_and_none_equivariant_packed1d_not():
    """The failure mode of the abstract at the operator level: the same physical data under
    another packing gives the permuted outputs with grid-coordinate RoPE (and with no
    rotation), and different outputs with packed-position RoPE."""
    w = si.small_workload(grid=(4, 4, 8), block=(2, 2, 2), radius=1, heads=2, head_dim=12, seed=33)
    res = {}
    for packing in ("raster", "random"):
        x = si.make_inputs(w, torch.float32, packing=packing)
        inv = np.argsort(x["perm"][0].numpy())               # raster index -> packed position
        for mode in oracle.pack3d.POSITION_MODES:
            o, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1, position_mode=mode)
            res[(packing, mode)] = o[0][inv]                 # back to raster order
    for mode in ("axial", "none"):
        np.testing.assert_allclose(res[("random", mode)], res[("raster", mode)], atol=1e-12)
    assert np.abs(res[("random", "packed1d")] - res[("raster", "packed1d")]).max() > 1e-2


def _torch_rope_1d(x, base):
    """1D RoPE at positions 0..N-1 through torch complex arithmetic."""
    n, h, d = x.shape
    z = torch.complex(x[..., : d // 2], x[..., d // 2:])
    freq = torch.exp(math.log(base) * (-torch.arange(d // 2, dtype=torch.float64) * 2.0 / d))
    w = torch.polar(torch.ones(n, d // 2, dtype=torch.float64), torch.arange(n, dtype=torch.float64)[:, None] * freq)
    zr = z * w[:, None, :]
    return torch.cat([zr.real, zr.imag], -1)


@pytest.mark.parametrize("mode", ["none", "packed1d"])
def test_backward_against_autograd(mode):
    w = si.small_workload(grid=(4, 4, 6), block=(2, 2, 2), radius=1, heads=2, head_dim=12, packing="random",
                          seed=34)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1, position_mode=mode)
    rot = (lambda t: t) if mode == "none" else (lambda t: _torch_rope_1d(t, 10000.0))
    q, k, v = (x[n][0].double().clone().requires_grad_() for n in ("q", "k", "v"))
    o = dense_masked(q, k, v, x["coords"][0].long(), w.block, 1, rot)
    (o * x["do"][0].double()).sum().backward()
    for g, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(g[0], ref.numpy(), atol=1e-11)
