"""Plain fp64 CPU oracle of a pre-norm transformer block around the PACK3D operator.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the CPU-baseline leg of
``bench.py``; never by the HIP library.

"Geometry Matters in Packed 3D Attention" (abstract) presents the operator as a
trainable attention layer for packed 3D data; the pages give no block layout.
Reading (the plainest one): a standard pre-norm transformer block whose
attention is PACK3D, with one fused QKV projection (columns ordered
(q|k|v, head, dim)), no projection biases, LayerNorm with affine weights, and a
GELU MLP of hidden width ``mlp_ratio * C``:

    h   = LN(x; g1, b1)
    qkv = h W_qkv^T            -> q, k, v [T, H, D] (column s C + h D + d)
    a   = PACK3D(q, k, v)       (oracle.pack3d.forward / backward, fp64)
    x1  = x + a W_o^T
    y   = x1 + GELU(LN(x1; g2, b2) W_1^T) W_2^T

LN(z) = (z - mean(z)) / sqrt(var(z) + 1e-5) * g + b over the channel dim, var
the biased variance; GELU(u) = u Phi(u) = u (1 + erf(u / sqrt 2)) / 2.
Everything else (locality, summaries, RoPE) is the operator of oracle.pack3d.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import pack3d as op

LN_EPS = 1e-5


class _Pack3DOracle(torch.autograd.Function):
    """The oracle operator as an autograd step: forward by oracle.pack3d.forward, backward by
    oracle.pack3d.backward (both fp64 NumPy)."""

    @staticmethod
    def forward(ctx, q, k, v, coords, block_shape, radius, rope_base, offsets, ragged):
        o, _ = op.forward(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), coords, block_shape, radius,
                          rope_base=rope_base, offsets=offsets, ragged=ragged)
        ctx.save_for_backward(q, k, v)
        ctx.args = (coords, block_shape, radius, rope_base, offsets, ragged)
        return torch.from_numpy(o)

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        coords, block_shape, radius, rope_base, offsets, ragged = ctx.args
        dq, dk, dv = op.backward(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), coords,
                                 do.detach().numpy(), block_shape, radius, rope_base=rope_base, offsets=offsets,
                                 ragged=ragged)
        return (torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv), None, None, None, None, None, None)


def layer_norm(z, g, b):
    mu = z.mean(-1, keepdim=True)
    var = ((z - mu) ** 2).mean(-1, keepdim=True)
    return (z - mu) / torch.sqrt(var + LN_EPS) * g + b


def gelu(u):
    return 0.5 * u * (1.0 + torch.erf(u / math.sqrt(2.0)))


def init_params(dim: int, mlp_ratio: int = 4, seed: int = 0) -> dict:
    """Seeded fp64 weights (LayerNorm weights near 1 and biases near 0, projections ~ N(0, 1/fan_in))."""
    g = np.random.default_rng(seed)

    def lin(out_f, in_f):
        return torch.from_numpy(g.standard_normal((out_f, in_f)) / math.sqrt(in_f))

    def vec(n, center, spread):
        return torch.from_numpy(center + spread * g.standard_normal(n))

    hid = mlp_ratio * dim
    return {"ln1_w": vec(dim, 1.0, 0.1), "ln1_b": vec(dim, 0.0, 0.1), "qkv": lin(3 * dim, dim),
            "proj": lin(dim, dim), "ln2_w": vec(dim, 1.0, 0.1), "ln2_b": vec(dim, 0.0, 0.1),
            "fc1": lin(hid, dim), "fc2": lin(dim, hid)}


def block_forward(x, params: dict, coords, block_shape, radius: int, heads: int, *, rope_base=10000.0,
                  attention=None, offsets=None, ragged=False):
    """y for x [B, N, C] (or flat [T, C] with ``offsets``), fp64 torch with autograd.

    ``attention(q, k, v)`` replaces the operator (default: the oracle PACK3D step); q, k, v
    are [B, N, H, D] (or [T, H, D]) fp64 tensors.
    """
    c = x.shape[-1]
    d = c // heads
    lead = x.shape[:-1]
    h = layer_norm(x, params["ln1_w"], params["ln1_b"])
    qkv = h @ params["qkv"].T
    q, k, v = (qkv[..., s * c:(s + 1) * c].reshape(*lead, heads, d) for s in range(3))
    if attention is None:
        a = _Pack3DOracle.apply(q, k, v, np.asarray(coords), tuple(block_shape), int(radius), float(rope_base),
                                offsets, ragged)
    else:
        a = attention(q, k, v)
    x1 = x + a.reshape(*lead, c) @ params["proj"].T
    m = gelu(layer_norm(x1, params["ln2_w"], params["ln2_b"]) @ params["fc1"].T) @ params["fc2"].T
    return x1 + m
