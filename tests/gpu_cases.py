"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3

DEV = "cuda:0"
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}   # max-abs error on o, dq, dk, dv


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in x.items()}


def gpu_forward(w, dtype, x=None, with_summaries=True, keep_workspace=False, **kw):
    """Returns (inputs on CPU, index, out, lse, workspace)."""
    if x is None:
        x = si.make_inputs(w, dtype, **kw)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    attn = p3.make_attn(dtype, w.heads, w.head_dim, w.rope_base, with_summaries=with_summaries)
    ws = torch.empty(p3.workspace_bytes(ix, attn), dtype=torch.uint8, device=DEV)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base,
                          with_summaries=with_summaries, workspace=ws)
    torch.cuda.synchronize()
    return x, ix, out, lse, ws


def max_err(gpu, ref, mask=None):
    g = gpu.detach().float().cpu().double().numpy()
    if mask is not None:
        g, ref = g[mask], ref[mask]
    return float(np.abs(g - ref).max())


def sample_blocks(nb, count=12, seed=0):
    """Corner, edge and interior blocks plus random ones (block ids, raster over the block grid)."""
    nbz, nby, nbx = nb
    ids = {0, nbz * nby * nbx - 1, nbx - 1, (nby - 1) * nbx, (nbz // 2 * nby + nby // 2) * nbx + nbx // 2,
           ((nbz - 1) * nby) * nbx + nbx // 2}
    rng = np.random.default_rng(seed)
    while len(ids) < count:
        ids.add(int(rng.integers(0, nbz * nby * nbx)))
    return sorted(ids)
