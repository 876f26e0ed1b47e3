"""Pins of the oracle's axial RoPE.

Convention: three contiguous head-dim groups (z, y, x) of width d_a = D/3;
half-split pairs (k, k + d_a/2); theta_k = base^(-2k/d_a); (x1, x2) ->
(x1 cos - x2 sin, x1 sin + x2 cos).  This is the rotation of the
"SpatioTemporal RoPE" section of the HorizonStream post applied per axis, with
three axes; "Geometry Matters in Packed 3D Attention" (abstract) fixes that the
angles come from the true grid coordinates.
"""
import math

import numpy as np
import pytest

import oracle


def test_closed_form_single_pair_per_axis():
    """D = 6: one pair per axis, theta_0 = 1, so e_(2a) turns to (cos c_a, sin c_a)."""
    coords = np.array([[1, 2, 3]])
    x = np.array([[1.0, 0.0, 1.0, 0.0, 1.0, 0.0]])
    got = oracle.rope(x, coords, base=10000.0)[0]
    want = [math.cos(1), math.sin(1), math.cos(2), math.sin(2), math.cos(3), math.sin(3)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_closed_form_half_split_pairing_and_frequencies():
    """D = 12: per axis theta = (1, base^(-1/2)); element k pairs with k + 2."""
    base = 10000.0
    c = np.array([[3, 5, 7]])
    for axis in range(3):
        for k in range(2):
            x = np.zeros((1, 12))
            x[0, 4 * axis + k] = 1.0
            got = oracle.rope(x, c, base=base)[0]
            phi = c[0, axis] * (1.0, base ** -0.5)[k]
            want = np.zeros(12)
            want[4 * axis + k] = math.cos(phi)
            want[4 * axis + k + 2] = math.sin(phi)
            assert np.allclose(got, want, rtol=0, atol=1e-15), (axis, k)
    # the partner element turns the other way: e_(k+2) -> (-sin, cos)
    x = np.zeros((1, 12))
    x[0, 2] = 1.0
    got = oracle.rope(x, c, base=base)[0]
    want = np.zeros(12)
    want[0], want[2] = -math.sin(3.0), math.cos(3.0)
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_frequencies():
    assert np.allclose(oracle.rope_tables(16, 10000.0), 10000.0 ** (-np.arange(0, 16, 2) / 16.0))
    assert oracle.rope_tables(32, 10000.0)[0] == 1.0


def test_identity_norm_relative_and_inverse():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 96))
    y = rng.standard_normal((50, 3, 96))
    a = rng.integers(-40, 40, size=(50, 3))
    b = rng.integers(-40, 40, size=(50, 3))
    assert np.array_equal(oracle.rope(x, np.zeros((50, 3), int)), x)
    rx = oracle.rope(x, a)
    assert np.allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    lhs = (oracle.rope(x, a) * oracle.rope(y, b)).sum(-1)
    rhs = (x * oracle.rope(y, b - a)).sum(-1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-12)
    assert np.allclose(oracle.rope(rx, a, inverse=True), x, rtol=0, atol=1e-13)


def test_rejects_bad_head_dim():
    with pytest.raises(ValueError):
        oracle.rope(np.zeros((1, 8)), np.zeros((1, 3)))
