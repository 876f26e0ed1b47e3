"""The oracle's pins have power: planted mistakes and negative controls fail them.

Each test plants one plausible mistake in the oracle (on the CPU, through
monkeypatch) or builds a deliberately wrong variant, then shows that a pin
from the other oracle test files rejects it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.pack3d as op
import synthetic_inputs as si
from tests.test_oracle_backward import _dense_masked
from tests.test_oracle_forward import _sdpa_reference


def _w(**kw):
    base = dict(grid=(4, 6, 8), block=(2, 2, 2), head_dim=12, heads=2, seed=41)
    base.update(kw)
    return si.small_workload(**base)


def _q0_closed_form_error(w):
    x = si.make_inputs(w, torch.float32)
    q0 = torch.zeros_like(x["q"])
    o, _ = oracle.forward(q0, x["k"], x["v"], x["coords"], w.block, 1)
    cn, vn = x["coords"][0].numpy(), x["v"][0].double().numpy()
    bc = (cn - cn.min(0)) // np.array(w.block)
    keys = {tuple(b) for b in bc.tolist()}
    err = 0.0
    for i in range(0, cn.shape[0], 11):
        loc = np.abs(bc - bc[i]).max(1) <= 1
        far = [b for b in keys if max(abs(a - bb) for a, bb in zip(b, bc[i])) > 1]
        total = vn[loc].sum(0) + sum(vn[(bc == np.array(b)).all(1)].mean(0) for b in far)
        err = max(err, np.abs(o[0, i] - total / (loc.sum() + len(far))).max())
    return err


def test_sum_instead_of_mean_pooling_fails_closed_form(monkeypatch):
    w = _w()
    assert _q0_closed_form_error(w) < 1e-13
    monkeypatch.setattr(op, "pool_blocks", lambda x, b, count=None: x.reshape(x.shape[0] // b, b, *x.shape[1:]).sum(1))
    assert _q0_closed_form_error(w) > 1e-3


def test_dropped_summaries_fail_closed_form_and_unit_block_reduction(monkeypatch):
    w = _w()
    monkeypatch.setattr(op, "_summary_blocks", lambda ix, qb, local: np.zeros(0, dtype=np.int64))
    assert _q0_closed_form_error(w) > 1e-3
    w1 = _w(grid=(4, 4, 6), block=(1, 1, 1))
    x = si.make_inputs(w1, torch.float32)
    od, _ = _sdpa_reference(x["q"], x["k"], x["v"], x["coords"], w1.rope_base)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w1.block, 1)
    assert np.abs(o - od).max() > 1e-3


def test_missing_own_block_fails_naive_agreement(monkeypatch):
    w = _w()
    x = si.make_inputs(w, torch.float32)
    ref, _ = oracle.forward_naive(x["q"], x["k"], x["v"], x["coords"], w.block, 1)
    orig = op._local_blocks
    monkeypatch.setattr(op, "_local_blocks", lambda ix, qb: [b for b in orig(ix, qb) if b != qb])
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1)
    assert np.abs(o - ref).max() > 1e-3


def test_wrong_rope_direction_or_pairing_fails_closed_forms(monkeypatch):
    coords = np.array([[1, 2, 3]])
    x = np.zeros((1, 12))
    x[0, 0] = 1.0
    want = np.zeros(12)
    want[0], want[2] = math.cos(1.0), math.sin(1.0)
    assert np.allclose(oracle.rope(x, coords), want, atol=1e-15)
    # rotation in the other direction
    assert not np.allclose(oracle.rope(x, coords, inverse=True), want, atol=1e-3)
    # interleaved pairing (k with k+1) instead of half-split
    def interleaved(x, c, base=10000.0, inverse=False):
        x = np.asarray(x, dtype=np.float64)
        out = x.copy()
        theta = op.rope_tables(x.shape[-1] // 3, base)
        for a in range(3):
            for kk, th in enumerate(theta):
                i, j = a * x.shape[-1] // 3 + 2 * kk, a * x.shape[-1] // 3 + 2 * kk + 1
                phi = np.asarray(c, dtype=float)[:, a] * th
                out[..., i] = x[..., i] * np.cos(phi) - x[..., j] * np.sin(phi)
                out[..., j] = x[..., i] * np.sin(phi) + x[..., j] * np.cos(phi)
        return out
    assert not np.allclose(interleaved(x, coords), want, atol=1e-3)


def test_dropped_pooling_gradient_fails_autograd(monkeypatch):
    w = _w(grid=(4, 4, 8), head_dim=12, heads=1)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    q = x["q"][0].double().requires_grad_()
    k = x["k"][0].double().requires_grad_()
    v = x["v"][0].double().requires_grad_()
    o = _dense_masked(q, k, v, x["coords"][0].long(), w.block, 1, w.rope_base)
    (o * x["do"][0].double()).sum().backward()
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    assert np.abs(dk[0] - k.grad.numpy()).max() < 1e-12
    # plant: the summary gradients are never broadcast back to the block members
    monkeypatch.setattr(op, "unpool_grad", lambda dbar, bvol, count=None: np.zeros((dbar.shape[0] * bvol,) + dbar.shape[1:]))
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    assert np.abs(dk[0] - k.grad.numpy()).max() > 1e-6 and np.abs(dv[0] - v.grad.numpy()).max() > 1e-6


def test_skipped_rope_transpose_fails_autograd(monkeypatch):
    w = _w(grid=(2, 4, 4), block=(1, 2, 2), head_dim=6, heads=1)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    q = x["q"][0].double().requires_grad_()
    k = x["k"][0].double().requires_grad_()
    v = x["v"][0].double().requires_grad_()
    o = _dense_masked(q, k, v, x["coords"][0].long(), w.block, 1, w.rope_base)
    (o * x["do"][0].double()).sum().backward()
    # plant: the RoPE transpose is skipped on the way back (dq = dQ~)
    monkeypatch.setattr(op, "rope", _rope_forward_only)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, 1)
    assert np.abs(dq[0] - q.grad.numpy()).max() > 1e-6


_true_rope = op.rope


def _rope_forward_only(x, coords, base=10000.0, inverse=False):
    return np.asarray(x, dtype=np.float64).copy() if inverse else _true_rope(x, coords, base)


def test_negative_control_packed_sequence_rope_breaks_repacking_equivariance():
    """(a) RoPE on the packed 1D position instead of the grid coordinates: outputs change with packing."""
    w = _w()
    outs = []
    for packing in ("raster", "random"):
        x = si.make_inputs(w, torch.float32, packing=packing)
        n = x["coords"].shape[1]
        seq = np.zeros((1, n, 3), dtype=np.int64)
        seq[0, :, 2] = np.arange(n)
        o, _ = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, 1, rope_coords=seq)
        outs.append(o[0][np.argsort(x["perm"][0].numpy())])
    assert np.abs(outs[0] - outs[1]).max() > 1e-3


def test_negative_control_pool_then_rotate_breaks_identity():
    """(b) Pooling unrotated keys and rotating the mean by the block centroid is not the summary."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((8, 12))
    c = np.array([[z, y, x] for z in (4, 5) for y in (2, 3) for x in (6, 7)])
    rotate_then_pool = oracle.rope(k, c).mean(0)
    pool_then_rotate = oracle.rope(k.mean(0)[None], c.mean(0)[None])[0]
    assert np.abs(rotate_then_pool - pool_then_rotate).max() > 1e-2


def test_negative_control_lattice_anchored_at_zero_breaks_shift_invariance():
    """(c) Anchoring the block lattice at absolute 0 regroups tokens under a shift that is not a
    multiple of the block; anchoring at the volume's minimum (the oracle's reading) does not."""
    grid, block = (4, 4, 4), np.array([2, 2, 2])
    c = si.raster_coords(grid).astype(np.int64)
    shifted = c + np.array([1, 0, 0])
    groups = lambda bc: {frozenset(np.nonzero((bc == b).all(1))[0].tolist()) for b in np.unique(bc, axis=0)}
    assert groups(c // block) != groups(shifted // block)
    ia = oracle.build_index(c[None], tuple(block), 1)[0]
    ib = oracle.build_index(shifted[None], tuple(block), 1)[0]
    assert np.array_equal(ia["token_block"], ib["token_block"])


# ---- ragged geometry -------------------------------------------------------------

def _ragged_naive_error():
    x = si.make_ragged_inputs([(5, 6, 7)], 2, 12, occupancy=0.6, seed=61)
    args = (x["q"][None], x["k"][None], x["v"][None], x["coords"][None], (2, 2, 2), 1)
    o, _ = oracle.forward(*args, ragged=True)
    o2, _ = oracle.forward_naive(*args)
    return np.abs(o - o2).max()


def test_pooling_over_whole_block_volume_fails_ragged_definition(monkeypatch):
    """Dividing a partial block's sum by |b| instead of the tokens present."""
    assert _ragged_naive_error() < 1e-12
    orig = op.pool_blocks
    monkeypatch.setattr(op, "pool_blocks", lambda x, b, count=None: orig(x, b))
    assert _ragged_naive_error() > 1e-3


def test_empty_block_summaries_fail_ragged_definition(monkeypatch):
    """Giving empty blocks a (zero) summary logit."""
    monkeypatch.setattr(op, "_summary_blocks",
                        lambda ix, qb, local: np.setdiff1d(np.arange(ix["nblk"]), np.asarray(local, dtype=np.int64)))
    assert _ragged_naive_error() > 1e-3


def test_absent_keys_left_in_local_set_fail_ragged_definition(monkeypatch):
    """Keeping the empty slots of the local blocks as (zero) keys."""
    orig = op._key_rows
    monkeypatch.setattr(op, "_key_rows", lambda local, bvol, present=None: orig(local, bvol))
    assert _ragged_naive_error() > 1e-3


def test_unpool_by_block_volume_fails_ragged_autograd(monkeypatch):
    from tests.dense_ref import dense_masked
    x = si.make_ragged_inputs([(5, 4, 7)], 2, 12, occupancy=0.7, seed=62, with_grad=True)
    orig = op.unpool_grad
    monkeypatch.setattr(op, "unpool_grad", lambda dbar, bvol, count=None: orig(dbar, bvol))
    _, dk, _ = oracle.backward(x["q"][None], x["k"][None], x["v"][None], x["coords"][None], x["do"][None],
                               (2, 2, 3), 1, ragged=True, position_mode="none")
    q, k, v = (x[n].double().clone().requires_grad_() for n in ("q", "k", "v"))
    o = dense_masked(q, k, v, x["coords"].long(), (2, 2, 3), 1, lambda t: t)
    (o * x["do"].double()).sum().backward()
    assert np.abs(dk[0] - k.grad.numpy()).max() > 1e-4


def test_unscaled_or_unrotated_gradients_fail_conservation(monkeypatch):
    from tests.test_oracle_backward import _conservation
    w = _w(grid=(4, 4, 8), head_dim=12, heads=2)
    x = si.make_inputs(w, torch.float32, with_grad=True)
    do = x["do"] + 0.75
    args = (x["q"], x["k"], x["v"], x["coords"], do, w.block, 1)
    gap, rot = _conservation(*args)[0]
    assert np.abs(gap).max() < 1e-11 and np.abs(rot).max() < 1e-11
    with monkeypatch.context() as m:
        # plant: every block member receives the whole summary gradient (no 1/n_b)
        m.setattr(op, "unpool_grad", lambda dbar, bvol, count=None: np.repeat(dbar, bvol, axis=0))
        gap, rot = _conservation(*args)[0]
        assert np.abs(gap).max() > 1e-3 and np.abs(rot).max() > 1e-3
    with monkeypatch.context() as m:
        m.setattr(op, "rope", _rope_forward_only)       # plant: RoPE transpose skipped on the way back
        gap, rot = _conservation(*args)[0]
        assert np.abs(gap).max() < 1e-11 and np.abs(rot).max() > 1e-3
