"""Plain fp64 NumPy oracle of PACK3D (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the HIP library.

What is computed ("Geometry Matters in Packed 3D Attention", abstract):

* A packed volume is a sequence of tokens, each carrying its true integer
  grid coordinate (z, y, x).  The packing order is arbitrary; only the
  coordinates define geometry.
* The volume is cut into contiguous 3D blocks of shape (bz, by, bx).  Reading
  (block-granular locality): a query attends exactly to every key whose block
  lies within Chebyshev distance ``r`` (in block units) of the query's block,
  truncated at the volume edge, and to one summary per remaining block of the
  same volume.
* Axial RoPE on the true grid coordinates rotates Q and K, head dim split into
  three contiguous groups (z, y, x).  Within a group of width d_a the pairs are
  (k, k + d_a/2), with frequency theta_k = base^(-2k/d_a), the same set on
  every axis (the convention of the "SpatioTemporal RoPE" section of the
  HorizonStream post, reduced to three axes).
* The rotation is applied before a block is summarized: the block summary is
  the mean of the block's *rotated* keys and the mean of its values, so a
  query-summary logit is the mean of that query's logits to the block's keys.
* Local logits and summary logits share one softmax (scale 1/sqrt(D) unless
  given).

Position modes (controls).  The abstract contrasts axial RoPE on grid
coordinates with position encodings indexed by the packed sequence, which
break under repacking.  ``position_mode`` selects the angle source of the same
operator: "axial" (the method), "packed1d" (standard RoPE on the packed
sequence position: the rotation of the RoPE section applied to the whole head
dim, pairs (k, k + D/2), theta_k = base^(-2k/D), angle = packed index * theta_k)
and "none" (no rotation).  Locality and summaries always follow the grid.

Ragged geometry (``ragged=True``).  The abstract speaks of packed geometric
data in general; a volume is then any set of distinct integer points (holes,
extents that the block does not divide).  Plainest reading, used here: the
block lattice is still anchored at the componentwise minimum and covers the
bounding box with ceil(extent / b) blocks per axis; a block holds the tokens
present in it; the local set is the present tokens of the blocks within the
radius; every other *occupied* block gives one summary, the mean over the
tokens present in it; an empty block gives none.  Canonical order keeps |b|
slots per block, an absent point leaving its slot empty (perm = -1).  A batch
of volumes with different token counts is passed flat ([T, H, D], coords
[T, 3]) with ``offsets`` [B + 1]; lse is then [B, H, max N_v], NaN past N_v.

Readings where the pages are silent (each listed in the design notes):
block lattice anchored at each volume's componentwise minimum coordinate; by
default only full grids with extents divisible by the block are accepted; no
causal mask; V is not rotated; lse is the natural-log log-sum-exp of the scaled
logits; gradients are taken with respect to the unrotated q, k, v.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


class CoordsError(ValueError):
    """Invalid geometry: ``reason`` in {"grid", "divisible", "duplicate"}."""

    def __init__(self, volume: int, reason: str, token: int = -1):
        super().__init__(f"volume {volume}: {reason} (token {token})")
        self.volume, self.reason, self.token = volume, reason, token


# --------------------------------------------------------------------------
# Index: block membership, canonical order, neighbour table
# --------------------------------------------------------------------------

def _volume_index(c: np.ndarray, block, r: int, volume: int, ragged: bool = False) -> dict:
    """Tables of one volume.  ``c`` int [N, 3] (z, y, x).

    ``perm`` [nblk * |b|] maps a canonical slot to the packed position of its token, -1
    for an empty slot (ragged geometry only); ``count`` [nblk] is the number of tokens
    present in each block."""
    c = c.astype(np.int64)
    n = c.shape[0]
    b = np.asarray(block, dtype=np.int64)
    if n == 0:
        raise CoordsError(volume, "empty")
    origin = c.min(axis=0)
    extent = c.max(axis=0) - origin + 1
    if not ragged:
        if int(np.prod(extent)) != n:
            raise CoordsError(volume, "grid")
        if np.any(extent % b):
            raise CoordsError(volume, "divisible")
    rel = c - origin
    # Duplicates: a token is offending when an earlier token has the same point.
    _, first_idx, inv = np.unique(rel, axis=0, return_index=True, return_inverse=True)
    dup = np.nonzero(first_idx[inv.reshape(-1)] != np.arange(n))[0]
    if dup.size:
        raise CoordsError(volume, "duplicate", int(dup.min()))
    nb = -(-extent // b)                                    # ceil: partial edge blocks
    bvol = int(np.prod(b))
    beta = rel // b
    blk = (beta[:, 0] * nb[1] + beta[:, 1]) * nb[2] + beta[:, 2]
    w = rel - beta * b
    omega = (w[:, 0] * b[1] + w[:, 1]) * b[2] + w[:, 2]
    canon = blk * bvol + omega
    nblk = int(np.prod(nb))
    perm = np.full(nblk * bvol, -1, dtype=np.int64)
    perm[canon] = np.arange(n)
    count = np.bincount(blk, minlength=nblk)
    offsets = list(itertools.product(range(-r, r + 1), repeat=3))  # (dz, dy, dx) raster
    nbr = np.full((nblk, len(offsets)), -1, dtype=np.int64)
    for bid in range(nblk):
        bz, rem = divmod(bid, int(nb[1] * nb[2]))
        by, bx = divmod(rem, int(nb[2]))
        for s, (dz, dy, dx) in enumerate(offsets):
            z, y, x = bz + dz, by + dy, bx + dx
            if 0 <= z < nb[0] and 0 <= y < nb[1] and 0 <= x < nb[2]:
                nbr[bid, s] = (z * nb[1] + y) * nb[2] + x
    return dict(origin=origin, extent=extent, nb=nb, nblk=nblk, bvol=bvol, block=b, n=n,
                token_block=blk, canon=canon, perm=perm, count=count, present=perm >= 0, nbr=nbr,
                radius=r)


def split_volumes(x, offsets=None) -> list:
    """Per-volume arrays: x [B, N, ...] (offsets None) or flat x [T, ...] cut at offsets [B + 1]."""
    if offsets is None:
        return [x[v] for v in range(x.shape[0])]
    off = [int(o) for o in offsets]
    if off[0] != 0 or any(b < a for a, b in zip(off, off[1:])) or off[-1] != x.shape[0]:
        raise ValueError("offsets must start at 0, not decrease and end at the token count")
    return [x[a:b] for a, b in zip(off, off[1:])]


def build_index(coords, block_shape, local_radius: int, *, ragged: bool = False, offsets=None) -> list:
    """Per-volume tables for coords int [B, N, 3] (z, y, x), or flat [T, 3] with ``offsets``.

    Raises ``CoordsError`` for the first bad volume (without ``ragged``: not a full
    grid, extents not divisible by the block; always: duplicate points, an empty
    volume) and ``ValueError`` for a bad block shape or a negative radius.
    """
    coords = np.asarray(coords)
    if coords.ndim == 2 and offsets is None:
        coords = coords[None]
    if len(block_shape) != 3 or min(block_shape) <= 0:
        raise ValueError("block_shape must hold three positive extents")
    if local_radius < 0:
        raise ValueError("local_radius must be >= 0")
    return [_volume_index(c, block_shape, int(local_radius), v, ragged)
            for v, c in enumerate(split_volumes(coords, offsets))]


# --------------------------------------------------------------------------
# Axial RoPE
# --------------------------------------------------------------------------

def rope_tables(d_axis: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/d_a), k = 0 .. d_a/2 - 1 (same set on every axis)."""
    if d_axis % 2:
        raise ValueError("per-axis width must be even")
    k = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / d_axis)


def rope(x, coords, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotate x [N, H, D] (or [N, D]) by the axial RoPE of coords [N, 3].

    Head dim = three contiguous groups (z, y, x) of width d_a = D/3; inside a
    group, element k pairs with element k + d_a/2 and turns by angle
    coord_a * theta_k:  (x1, x2) -> (x1 cos - x2 sin, x1 sin + x2 cos).
    ``inverse`` applies the transpose (rotation by minus the angle).
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    d = x.shape[-1]
    if d % 6:
        raise ValueError("head_dim must split into three even axis groups")
    da, half = d // 3, d // 6
    theta = rope_tables(da, base)
    c = np.asarray(coords, dtype=np.float64)
    sign = -1.0 if inverse else 1.0
    out = np.empty_like(x)
    for a in range(3):
        phi = c[:, a, None] * theta[None, :]           # [N, half]
        cos = np.cos(phi)[:, None, :]
        sin = sign * np.sin(phi)[:, None, :]
        x1 = x[..., a * da: a * da + half]
        x2 = x[..., a * da + half: (a + 1) * da]
        out[..., a * da: a * da + half] = x1 * cos - x2 * sin
        out[..., a * da + half: (a + 1) * da] = x1 * sin + x2 * cos
    return out[:, 0, :] if squeeze else out


def rope_1d(x, pos, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotate x [N, H, D] (or [N, D]) by standard 1D RoPE at integer positions pos [N].

    The whole head dim is one group: element k pairs with element k + D/2 and turns
    by angle pos * theta_k with theta_k = base^(-2k/D) ("SpatioTemporal RoPE"
    section: standard RoPE rotates by the 1D sequence position, half-split pairs).
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even")
    half = d // 2
    theta = rope_tables(d, base)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]    # [N, half]
    sign = -1.0 if inverse else 1.0
    cos = np.cos(phi)[:, None, :]
    sin = sign * np.sin(phi)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    out = np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)
    return out[:, 0, :] if squeeze else out


POSITION_MODES = ("axial", "packed1d", "none")


def rotate(x, coords, packed_pos, base: float, mode: str, inverse: bool = False) -> np.ndarray:
    """The rotation of ``mode``: axial RoPE on grid coordinates [N, 3], 1D RoPE on the
    packed sequence positions [N], or none."""
    if mode == "axial":
        return rope(x, coords, base, inverse)
    if mode == "packed1d":
        return rope_1d(x, packed_pos, base, inverse)
    if mode == "none":
        return np.array(x, dtype=np.float64)
    raise ValueError(f"unknown position mode {mode!r}")


def pool_blocks(x_canon: np.ndarray, bvol: int, count=None) -> np.ndarray:
    """Mean over the tokens present in each block of a canonical-order array [nblk * bvol, ...]
    whose empty slots hold zeros -> [nblk, ...]; an empty block gives zeros."""
    n = x_canon.shape[0]
    blocks = x_canon.reshape(n // bvol, bvol, *x_canon.shape[1:])
    if count is None:
        return blocks.mean(axis=1)
    cnt = np.asarray(count, dtype=np.float64).reshape(-1, *([1] * (x_canon.ndim - 1)))
    return np.divide(blocks.sum(axis=1), cnt, out=np.zeros_like(blocks[:, 0]), where=cnt > 0)


def unpool_grad(dbar: np.ndarray, bvol: int, count=None) -> np.ndarray:
    """Gradient of the block mean: every member of block b receives dbar_b / n_b (canonical order;
    n_b = |b| on a full grid, else the tokens present)."""
    if count is None:
        return np.repeat(dbar, bvol, axis=0) / bvol
    cnt = np.maximum(np.asarray(count, dtype=np.float64), 1.0).reshape(-1, *([1] * (dbar.ndim - 1)))
    return np.repeat(dbar / cnt, bvol, axis=0)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def _f64(t) -> np.ndarray:
    """Exact conversion of a numpy array or a CPU torch tensor to fp64 numpy."""
    if hasattr(t, "detach"):
        t = t.detach().to("cpu")
        import torch  # local: the oracle itself does not need torch
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _canonical(x, perm, present):
    """Rows of x [N, ...] in canonical order; empty slots hold zeros."""
    out = np.zeros((perm.shape[0], *x.shape[1:]), dtype=np.float64)
    out[present] = x[perm[present]]
    return out


def _prepare(q, k, v, coords, block_shape, r, base, rope_coords=None, position_mode="axial", ragged=False,
             offsets=None):
    q, k, v = _f64(q), _f64(k), _f64(v)
    coords = np.asarray(coords.numpy() if hasattr(coords, "numpy") else coords)
    if coords.ndim == 2 and offsets is None:
        coords = coords[None]
    index = build_index(coords, block_shape, r, ragged=ragged, offsets=offsets)
    rc = coords if rope_coords is None else np.asarray(rope_coords)
    qs, ks, vs, rcs = (split_volumes(x, offsets) for x in (q, k, v, rc))
    vols = []
    for vi, ix in enumerate(index):
        perm, present = ix["perm"], ix["present"]       # canonical slot -> packed position (-1: empty)
        pos = np.arange(ix["n"])
        qt = _canonical(rotate(qs[vi], rcs[vi], pos, base, position_mode), perm, present)
        kt = _canonical(rotate(ks[vi], rcs[vi], pos, base, position_mode), perm, present)
        vc = _canonical(vs[vi], perm, present)
        cnt = ix["count"] if ragged else None
        vols.append(dict(ix=ix, qt=qt, kt=kt, vc=vc,
                         kbar=pool_blocks(kt, ix["bvol"], cnt), vbar=pool_blocks(vc, ix["bvol"], cnt)))
    return q, k, v, coords, vols


def _local_blocks(ix, qb):
    return [int(n) for n in ix["nbr"][qb] if n >= 0]


def _summary_blocks(ix, qb, local):
    """Occupied blocks outside the local neighbourhood, in block-id order."""
    mask = ix["count"] > 0
    mask[local] = False
    return np.nonzero(mask)[0]


def _key_rows(local, bvol, present=None):
    rows = np.concatenate([np.arange(n * bvol, (n + 1) * bvol) for n in local])
    return rows if present is None else rows[present[rows]]


def _join(parts, offsets):
    """Per-volume arrays back to the caller's layout: stacked [B, N, ...] or flat [T, ...]."""
    return np.stack(parts) if offsets is None else np.concatenate(parts)


def forward(q, k, v, coords, block_shape, local_radius, *, rope_base=10000.0, scale=None,
            with_summaries=True, query_blocks=None, rope_coords=None, return_logits=False,
            position_mode="axial", ragged=False, offsets=None):
    """PACK3D forward.  q, k, v [B, N, H, D]; coords [B, N, 3] (z, y, x); or, with
    ``offsets`` [B + 1], flat q, k, v [T, H, D] and coords [T, 3].

    Returns (o, lse) in fp64, packed order: o shaped like q, lse [B, H, max N_v] (NaN
    past a volume's token count).  With ``query_blocks`` (a list of block ids) only
    those query blocks are computed in every volume; other rows are NaN.
    ``return_logits`` (tiny uniform inputs only) adds dense [B, H, N, N] local and
    [B, H, N, nblk] summary logit matrices, NaN where a pair is not in the set.
    ``position_mode`` picks the rotation and ``ragged`` admits any set of distinct
    points (see the module notes).
    """
    q, k, v, coords, vols = _prepare(q, k, v, coords, block_shape, local_radius, rope_base, rope_coords,
                                     position_mode, ragged, offsets)
    h, d = q.shape[-2], q.shape[-1]
    bsz = len(vols)
    nmax = max(vol["ix"]["n"] for vol in vols)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    outs = [np.full((vol["ix"]["n"], h, d), np.nan) for vol in vols]
    lse = np.full((bsz, h, nmax), np.nan)
    if return_logits:
        lg_loc = np.full((bsz, h, nmax, nmax), np.nan)
        lg_sum = np.full((bsz, h, nmax, max(vol["ix"]["nblk"] for vol in vols)), np.nan)
    for vi, vol in enumerate(vols):
        ix = vol["ix"]
        bvol, perm, present = ix["bvol"], ix["perm"], ix["present"]
        qbs = range(ix["nblk"]) if query_blocks is None else [qb for qb in query_blocks if qb < ix["nblk"]]
        for qb in qbs:
            rows = np.arange(qb * bvol, (qb + 1) * bvol)
            rows = rows[present[rows]]
            if rows.size == 0:
                continue
            local = _local_blocks(ix, qb)
            krows = _key_rows(local, bvol, present)
            qt = vol["qt"][rows].transpose(1, 0, 2)                          # [H, bq, D]
            s = scale * (qt @ vol["kt"][krows].transpose(1, 2, 0))           # [H, bq, nk]
            parts = [s]
            sb = _summary_blocks(ix, qb, local) if with_summaries else np.zeros(0, dtype=np.int64)
            use_sum = sb.size > 0
            if use_sum:
                t = scale * (qt @ vol["kbar"][sb].transpose(1, 2, 0))        # [H, bq, ns]
                parts.append(t)
            m = np.max(np.concatenate([p.max(axis=-1, keepdims=True) for p in parts], -1), -1, keepdims=True)
            es = np.exp(s - m)
            acc = es @ vol["vc"][krows].transpose(1, 0, 2)                   # [H, bq, D]
            den = es.sum(-1, keepdims=True)
            if use_sum:
                et = np.exp(t - m)
                acc = acc + et @ vol["vbar"][sb].transpose(1, 0, 2)
                den = den + et.sum(-1, keepdims=True)
            src = perm[rows]                                                 # packed positions
            outs[vi][src] = (acc / den).transpose(1, 0, 2)
            lse[vi][:, src] = (m + np.log(den))[..., 0]
            if return_logits:
                kp = perm[krows]
                lg_loc[vi][:, src[:, None], kp[None, :]] = s
                if use_sum:
                    lg_sum[vi][:, src[:, None], sb[None, :]] = t
    o = _join(outs, offsets)
    if return_logits:
        return o, lse, lg_loc, lg_sum
    return o, lse


def forward_naive(q, k, v, coords, block_shape, local_radius, *, rope_base=10000.0, scale=None,
                  with_summaries=True, position_mode="axial"):
    """The definition token by token, with no index tables (tiny inputs only).

    Membership is decided by brute force: key j is local to query i when the
    Chebyshev distance between their block coordinates is <= r; every other
    block of the volume contributes one summary, the mean of its rotated keys
    and of its values.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    coords = np.asarray(coords.numpy() if hasattr(coords, "numpy") else coords).astype(np.int64)
    bsz, n, h, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    b = np.asarray(block_shape, dtype=np.int64)
    o = np.zeros((bsz, n, h, d))
    lse = np.zeros((bsz, h, n))
    for vi in range(bsz):
        c = coords[vi]
        bc = (c - c.min(axis=0)) // b                      # block coordinate of every token
        pos = np.arange(n)                                 # tokens are in packed order here
        qt = rotate(q[vi], c, pos, rope_base, position_mode)
        kt = rotate(k[vi], c, pos, rope_base, position_mode)
        blocks = sorted({tuple(x) for x in bc.tolist()})
        members = {blk: np.nonzero((bc == np.asarray(blk)).all(axis=1))[0] for blk in blocks}
        kbar = {blk: kt[idx].mean(axis=0) for blk, idx in members.items()}
        vbar = {blk: v[vi][idx].mean(axis=0) for blk, idx in members.items()}
        for i in range(n):
            cheb_tok = np.abs(bc - bc[i]).max(axis=1)
            loc = np.nonzero(cheb_tok <= local_radius)[0]
            far = [blk for blk in blocks if max(abs(x - y) for x, y in zip(blk, bc[i])) > local_radius]
            for hh in range(h):
                logits = [scale * (kt[loc, hh] @ qt[i, hh])]
                vals = [v[vi][loc, hh]]
                if with_summaries and far:
                    logits.append(np.array([scale * (kbar[blk][hh] @ qt[i, hh]) for blk in far]))
                    vals.append(np.stack([vbar[blk][hh] for blk in far]))
                lg = np.concatenate(logits)
                vv = np.concatenate(vals)
                m = lg.max()
                e = np.exp(lg - m)
                o[vi, i, hh] = e @ vv / e.sum()
                lse[vi, hh, i] = m + np.log(e.sum())
    return o, lse


def dense_attention(q, k, v, coords, *, rope_base=10000.0, scale=None, position_mode="axial"):
    """Textbook softmax attention over every token of the volume, with the rotation of
    ``position_mode`` (3D RoPE by default)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    coords = np.asarray(coords.numpy() if hasattr(coords, "numpy") else coords)
    bsz, n, h, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.empty_like(q)
    lse = np.empty((bsz, h, n))
    for vi in range(bsz):
        pos = np.arange(n)
        qt = rotate(q[vi], coords[vi], pos, rope_base, position_mode).transpose(1, 0, 2)
        kt = rotate(k[vi], coords[vi], pos, rope_base, position_mode).transpose(1, 0, 2)
        s = scale * qt @ kt.transpose(0, 2, 1)
        m = s.max(-1, keepdims=True)
        e = np.exp(s - m)
        o[vi] = (e @ v[vi].transpose(1, 0, 2) / e.sum(-1, keepdims=True)).transpose(1, 0, 2)
        lse[vi] = (m + np.log(e.sum(-1, keepdims=True)))[..., 0]
    return o, lse


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def backward(q, k, v, coords, do, block_shape, local_radius, *, rope_base=10000.0, scale=None,
             with_summaries=True, volumes=None, heads=None, position_mode="axial", ragged=False, offsets=None,
             query_blocks=None):
    """Gradients (dq, dk, dv) fp64 of sum(o * do) w.r.t. unrotated q, k, v, shaped like q
    (layouts as in ``forward``).

    With o_i = (sum_j P_ij V_j + sum_b P_ib Vbar_b), P = exp(logit - lse_i):
      delta_i = <dO_i, o_i>
      dS_ij = P_ij (<dO_i, V_j> - delta_i),  dT_ib = P_ib (<dO_i, Vbar_b> - delta_i)
      dQ~_i = scale (sum_j dS_ij K~_j + sum_b dT_ib Kbar_b)
      dK~_j = scale sum_i dS_ij Q~_i + dKbar_b(j) / n_b,  dKbar_b = scale sum_i dT_ib Q~_i
      dV_j  = sum_i P_ij dO_i + dVbar_b(j) / n_b,         dVbar_b = sum_i P_ib dO_i
      dq = R(c)^T dQ~, dk = R(c)^T dK~  (the mean pooling broadcasts 1/n_b to the n_b
      tokens present in block b; n_b = |b| on a full grid).
    ``volumes`` / ``heads`` restrict the work (other entries are NaN); R is the rotation of
    ``position_mode``.  With ``query_blocks`` (block ids, as in ``forward``) only dq of
    those query blocks is returned: dk and dv need every query, so they are all NaN.
    """
    q, k, v, coords, vols = _prepare(q, k, v, coords, block_shape, local_radius, rope_base,
                                     position_mode=position_mode, ragged=ragged, offsets=offsets)
    dos = split_volumes(_f64(do), offsets)
    rcs = split_volumes(coords, offsets)
    h, d = q.shape[-2], q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    grads = [[np.full((vol["ix"]["n"], h, d), np.nan) for vol in vols] for _ in range(3)]
    vsel = range(len(vols)) if volumes is None else volumes
    hsel = np.arange(h) if heads is None else np.asarray(heads)
    for vi in vsel:
        vol = vols[vi]
        ix = vol["ix"]
        bvol, perm, nblk, present = ix["bvol"], ix["perm"], ix["nblk"], ix["present"]
        qt_all, kt_all, vc_all = vol["qt"][:, hsel], vol["kt"][:, hsel], vol["vc"][:, hsel]
        kbar, vbar = vol["kbar"][:, hsel], vol["vbar"][:, hsel]
        doc = _canonical(dos[vi], perm, present)[:, hsel]
        dqt = np.zeros_like(qt_all)
        dkt = np.zeros_like(kt_all)
        dvc = np.zeros_like(vc_all)
        dkbar = np.zeros_like(kbar)
        dvbar = np.zeros_like(vbar)
        qbs = range(nblk) if query_blocks is None else [qb for qb in query_blocks if qb < nblk]
        done = np.zeros(present.shape, dtype=bool)               # canonical rows whose dq was computed
        for qb in qbs:
            rows = np.arange(qb * bvol, (qb + 1) * bvol)
            rows = rows[present[rows]]
            if rows.size == 0:
                continue
            done[rows] = True
            local = _local_blocks(ix, qb)
            krows = _key_rows(local, bvol, present)
            qt = qt_all[rows].transpose(1, 0, 2)                 # [H, bq, D]
            kk = kt_all[krows].transpose(1, 0, 2)                # [H, nk, D]
            vv = vc_all[krows].transpose(1, 0, 2)
            dob = doc[rows].transpose(1, 0, 2)                   # [H, bq, D]
            s = scale * qt @ kk.transpose(0, 2, 1)
            logits = [s]
            sb = _summary_blocks(ix, qb, local) if with_summaries else np.zeros(0, dtype=np.int64)
            use_sum = sb.size > 0
            if use_sum:
                kb = kbar[sb].transpose(1, 0, 2)
                vb = vbar[sb].transpose(1, 0, 2)
                t = scale * qt @ kb.transpose(0, 2, 1)
                logits.append(t)
            m = np.max(np.concatenate([x.max(-1, keepdims=True) for x in logits], -1), -1, keepdims=True)
            den = sum(np.exp(x - m).sum(-1, keepdims=True) for x in logits)
            lse = m + np.log(den)
            p = np.exp(s - lse)
            ob = p @ vv
            if use_sum:
                pt = np.exp(t - lse)
                ob = ob + pt @ vb
            delta = (dob * ob).sum(-1, keepdims=True)            # [H, bq, 1]
            ds = p * (dob @ vv.transpose(0, 2, 1) - delta)
            dqb = ds @ kk
            # krows lists each key once, so fancy-index accumulation is exact
            dkt[krows] += (scale * ds.transpose(0, 2, 1) @ qt).transpose(1, 0, 2)
            dvc[krows] += (p.transpose(0, 2, 1) @ dob).transpose(1, 0, 2)
            if use_sum:
                dt = pt * (dob @ vb.transpose(0, 2, 1) - delta)
                dqb = dqb + dt @ kb
                dkbar[sb] += (scale * dt.transpose(0, 2, 1) @ qt).transpose(1, 0, 2)
                dvbar[sb] += (pt.transpose(0, 2, 1) @ dob).transpose(1, 0, 2)
            dqt[rows] = scale * dqb.transpose(1, 0, 2)
        cnt = ix["count"] if ragged else None
        dkt += unpool_grad(dkbar, bvol, cnt)
        dvc += unpool_grad(dvbar, bvol, cnt)
        live = np.nonzero(present)[0]                            # canonical slots holding a token
        src = perm[live]
        c = rcs[vi][src]
        dq_c = rotate(dqt[live], c, src, rope_base, position_mode, inverse=True)
        dk_c = rotate(dkt[live], c, src, rope_base, position_mode, inverse=True)
        for gi, (g, val) in enumerate(zip(grads, (dq_c, dk_c, dvc[live]))):
            tmp = np.full((ix["n"], len(hsel), d), np.nan)
            if query_blocks is None:
                tmp[src] = val
            elif gi == 0:
                keep = done[live]
                tmp[src[keep]] = val[keep]
            g[vi][:, hsel] = tmp
    return tuple(_join(g, offsets) for g in grads)
