"""Independent dense-masked formulation of the operator for gradient pins (torch, fp64).

The mean pooling is an averaging matrix over the tokens present in each block, locality
is a boolean mask over block coordinates, and local logits and summary logits share one
softmax ("Geometry Matters in Packed 3D Attention", abstract).  It builds no index
tables and shares no code with the oracle, so torch.autograd through it checks the
oracle's hand-written gradients.
"""
import math

import torch


def dense_masked(q, k, v, c, block, r, rot, with_summaries=True):
    """Independent dense-masked formulation (torch, fp64): pooling as an averaging matrix and
    one softmax over [local keys | summaries]; rot(x) applies the rotation."""
    n, h, d = q.shape
    cc = c - c.min(0).values
    bc = cc // torch.tensor(block)
    keys, inv = torch.unique(bc, dim=0, return_inverse=True)
    pool = torch.zeros(keys.shape[0], n, dtype=torch.float64)
    pool[inv, torch.arange(n)] = 1.0
    pool = pool / pool.sum(1, keepdim=True)
    loc = (bc[:, None, :] - bc[None, :, :]).abs().amax(-1) <= r
    far = (bc[:, None, :] - keys[None, :, :]).abs().amax(-1) > r
    if not with_summaries:
        far = torch.zeros_like(far)
    qt, kt = rot(q), rot(k)
    kbar = torch.einsum("bn,nhd->bhd", pool, kt)
    vbar = torch.einsum("bn,nhd->bhd", pool, v)
    s = torch.einsum("ihd,jhd->hij", qt, kt) / math.sqrt(d)
    t = torch.einsum("ihd,bhd->hib", qt, kbar) / math.sqrt(d)
    s = s.masked_fill(~loc[None], float("-inf"))
    t = t.masked_fill(~far[None], float("-inf"))
    p = torch.softmax(torch.cat([s, t], -1), -1)
    vals = torch.cat([v.transpose(0, 1), vbar.transpose(0, 1)], 1)
    return (p @ vals).transpose(0, 1)


def torch_axial_rope(x, c, base=10000.0):
    """Axial RoPE through torch complex arithmetic: per axis group of width d/3, the pair
    (k, k + d/6) is one complex number turned by exp(i c_axis base^(-2k/(d/3)))."""
    n, h, d = x.shape
    da, half = d // 3, d // 6
    freq = torch.exp(math.log(base) * (-torch.arange(half, dtype=torch.float64) * 2.0 / da))
    parts = []
    for a in range(3):
        g = x[..., a * da:(a + 1) * da]
        z = torch.complex(g[..., :half], g[..., half:])
        w = torch.polar(torch.ones(n, half, dtype=torch.float64), c[:, a, None].double() * freq)
        zr = z * w[:, None, :]
        parts += [zr.real, zr.imag]
    return torch.cat(parts, -1)
