"""Seeded synthetic inputs for the PACK3D operator.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark. It holds no arithmetic of the operator itself: it only lays out a
full 3D grid of token coordinates, orders those tokens into one of the packings
named in the abstract of "Geometry Matters in Packed 3D Attention"
(arXiv:2610.38694) -- raster, Morton, block-contiguous, random -- and draws
Q, K, V and the upstream gradient from numpy's seeded generator.

Recipe (the same for every workload):
  * ``g = numpy.random.default_rng(seed)``; Q, then K, then V are drawn with
    ``g.standard_normal((B, Z, Y, X, H, D), dtype=float32)`` in raster order,
    multiplied by the workload's input scale, then (for bf16) rounded
    float32 -> bfloat16 with round-to-nearest-even.
  * The upstream gradient dO is drawn the same way from
    ``default_rng(seed + 2000)``.
  * Coordinates are the integer (z, y, x) grid positions starting at 0.
  * Each volume v gets its own packing permutation ``perm`` (packed position
    -> raster index); a random packing draws it from
    ``default_rng(seed + 1000 + v)``.
  * Every tensor is returned in packed order: ``x_packed[b, p] =
    x_raster[b, perm_b[p]]``.  The same physical data therefore appears under
    every packing.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

PACKINGS = ("raster", "morton", "block", "random")


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    grid: tuple          # (Z, Y, X)
    packing: str
    heads: int
    head_dim: int
    block: tuple         # (bz, by, bx)
    radius: int
    dtypes: tuple        # torch dtypes the workload is run in
    seed: int
    input_scale: float = 1.0
    rope_base: float = 10000.0
    with_backward: bool = False
    description: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        z, y, x = self.grid
        return z * y * x


# The five workloads of the benchmark spec, with their sizes.
WORKLOADS = {
    "tiny": Workload("tiny", 1, (8, 8, 8), "raster", 2, 48, (2, 2, 2), 1,
                     (torch.float32,), seed=0,
                     description="1 volume 8x8x8, raster, 2 heads, D=48, 2x2x2 blocks, fp32"),
    "16k": Workload("16k", 1, (16, 32, 32), "morton", 8, 96, (4, 4, 4), 1,
                    (torch.float32, torch.bfloat16), seed=1, input_scale=1.0 / np.sqrt(96.0),
                    description="1 volume 16x32x32, Morton, 8 heads, D=96, 4x4x4 blocks"),
    "65k": Workload("65k", 2, (32, 32, 64), "random", 8, 96, (4, 4, 4), 1,
                    (torch.bfloat16,), seed=2,
                    description="2 volumes 32x32x64, random packing, 8 heads, D=96, 4x4x4 blocks"),
    "524k": Workload("524k", 1, (32, 128, 128), "block", 8, 96, (4, 8, 8), 1,
                     (torch.bfloat16,), seed=3,
                     description="1 volume 32x128x128, block-contiguous, 8 heads, D=96, 4x8x8 blocks"),
    "65k-train": Workload("65k-train", 2, (32, 32, 64), "random", 8, 96, (4, 4, 4), 1,
                          (torch.bfloat16,), seed=4, with_backward=True,
                          description="65k shapes, forward + backward"),
}


def raster_coords(grid) -> np.ndarray:
    """All integer (z, y, x) points of a Z x Y x X grid in raster order (x fastest)."""
    z, y, x = grid
    zz, yy, xx = np.meshgrid(np.arange(z), np.arange(y), np.arange(x), indexing="ij")
    return np.stack([zz.ravel(), yy.ravel(), xx.ravel()], axis=1).astype(np.int32)


def _morton_code(c: np.ndarray) -> np.ndarray:
    """3D bit interleave: x at bit 3k, y at bit 3k+1, z at bit 3k+2."""
    code = np.zeros(c.shape[0], dtype=np.uint64)
    for bit in range(21):
        for axis, shift in ((2, 0), (1, 1), (0, 2)):
            b = (c[:, axis].astype(np.uint64) >> np.uint64(bit)) & np.uint64(1)
            code |= b << np.uint64(3 * bit + shift)
    return code


def _block_contiguous_order(grid, block) -> np.ndarray:
    """Raster indices visited block by block (blocks in raster order, raster inside each)."""
    z, y, x = grid
    bz, by, bx = block
    if z % bz or y % by or x % bx:
        raise ValueError("block-contiguous packing needs extents divisible by the block")
    idx = np.arange(z * y * x).reshape(z // bz, bz, y // by, by, x // bx, bx)
    return idx.transpose(0, 2, 4, 1, 3, 5).reshape(-1)


def packing_permutation(grid, packing: str, *, block=None, seed: int = 0, volume: int = 0) -> np.ndarray:
    """perm[p] = raster index of the token stored at packed position p."""
    n = int(np.prod(grid))
    if packing == "raster":
        return np.arange(n, dtype=np.int64)
    if packing == "morton":
        return np.argsort(_morton_code(raster_coords(grid)), kind="stable").astype(np.int64)
    if packing == "block":
        return _block_contiguous_order(grid, block).astype(np.int64)
    if packing == "random":
        return np.random.default_rng(seed + 1000 + volume).permutation(n).astype(np.int64)
    raise ValueError(f"unknown packing {packing!r}")


def _draw(rng, shape, scale, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    t = torch.from_numpy(x)
    return t.to(dtype) if dtype != torch.float32 else t


def make_inputs(w: Workload, dtype=None, *, packing: str | None = None, with_grad: bool = False,
                shift=(0, 0, 0)):
    """Return a dict of CPU tensors in packed order for workload ``w``.

    keys: q, k, v (and do if ``with_grad``) [B, N, H, D] in ``dtype``;
    coords int32 [B, N, 3] (z, y, x) (plus ``shift``); perm int64 [B, N].
    """
    dtype = dtype or w.dtypes[0]
    packing = packing or w.packing
    b, n, h, d = w.batch, w.tokens, w.heads, w.head_dim
    rng = np.random.default_rng(w.seed)
    shape = (b, n, h, d)
    raster = [_draw(rng, shape, w.input_scale, dtype) for _ in range(3)]
    do_raster = _draw(np.random.default_rng(w.seed + 2000), shape, 1.0, dtype) if with_grad else None
    rc = raster_coords(w.grid) + np.asarray(shift, dtype=np.int32)
    perms = np.stack([packing_permutation(w.grid, packing, block=w.block, seed=w.seed, volume=v)
                      for v in range(b)])
    pt = torch.from_numpy(perms)
    out = {}
    for name, t in zip(("q", "k", "v"), raster):
        out[name] = torch.stack([t[v, pt[v]] for v in range(b)]).contiguous()
    if do_raster is not None:
        out["do"] = torch.stack([do_raster[v, pt[v]] for v in range(b)]).contiguous()
    out["coords"] = torch.from_numpy(np.stack([rc[perms[v]] for v in range(b)])).contiguous()
    out["perm"] = pt
    return out


def small_workload(grid=(4, 6, 8), block=(2, 2, 2), heads=2, head_dim=12, radius=1, packing="random",
                   seed=7, batch=1, input_scale=1.0, rope_base=10000.0) -> Workload:
    """An ad-hoc small workload for tests."""
    return Workload(f"small{grid}", batch, tuple(grid), packing, heads, head_dim, tuple(block), radius,
                    (torch.float32,), seed=seed, input_scale=input_scale, rope_base=rope_base)


def make_ragged_inputs(grids, heads, head_dim, dtype=torch.float32, *, occupancy=1.0, seed=0, with_grad=False,
                       shifts=None, input_scale=1.0):
    """Seeded ragged batch, flat in packed order (tokens of volume v at offsets[v]:offsets[v+1]).

    Volume v holds the points of a ``grids[v]`` box (any extents), each kept with
    probability ``occupancy`` (the box corners always, so the extents are exact), moved
    by ``shifts[v]``, in a random packing order.  Values are N(0, 1) (times
    ``input_scale``) drawn per kept point in raster order.

    keys: q, k, v (and do) [T, H, D] in ``dtype``; coords int32 [T, 3]; offsets int64
    [B + 1]; raster int64 [T] (raster index of each token inside its box).
    """
    rng = np.random.default_rng(seed)
    qs, ks, vs, dos, cs, rs, offs = [], [], [], [], [], [], [0]
    for v, grid in enumerate(grids):
        rc = raster_coords(grid).astype(np.int64)
        keep = rng.random(rc.shape[0]) < occupancy
        hi = np.asarray(grid) - 1
        corner = ((rc == 0) | (rc == hi)).all(axis=1)
        keep |= corner
        idx = np.nonzero(keep)[0]
        order = rng.permutation(idx.shape[0])
        idx = idx[order]
        n = idx.shape[0]
        shift = np.zeros(3, dtype=np.int64) if shifts is None else np.asarray(shifts[v], dtype=np.int64)
        cs.append((rc[idx] + shift).astype(np.int32))
        rs.append(idx)
        for lst in (qs, ks, vs):
            full = _draw(rng, (rc.shape[0], heads, head_dim), input_scale, dtype)
            lst.append(full[torch.from_numpy(idx)])
        if with_grad:
            full = _draw(np.random.default_rng(seed + 2000 + v), (rc.shape[0], heads, head_dim), 1.0, dtype)
            dos.append(full[torch.from_numpy(idx)])
        offs.append(offs[-1] + n)
    out = {"q": torch.cat(qs).contiguous(), "k": torch.cat(ks).contiguous(), "v": torch.cat(vs).contiguous(),
           "coords": torch.from_numpy(np.concatenate(cs)).contiguous(),
           "offsets": torch.tensor(offs, dtype=torch.int64), "raster": torch.from_numpy(np.concatenate(rs))}
    if with_grad:
        out["do"] = torch.cat(dos).contiguous()
    return out


# Ragged stand-ins for cropped, partly occupied microscopy volumes: two volumes of
# different shapes (extents not divisible by the block) with random holes, flat in a
# varlen batch; about 111k tokens in all, sized like the 65k-per-volume workload.
RAGGED_WORKLOADS = {
    "65k-ragged": dict(grids=[(30, 34, 62), (32, 30, 60)], occupancy=0.92, block=(4, 4, 4), radius=1, heads=8,
                       head_dim=96, seed=5, description="2 volumes 30x34x62 and 32x30x60 at 92% occupancy "
                       "(varlen, partial edge blocks, holes), 8 heads, D=96, 4x4x4 blocks"),
}
