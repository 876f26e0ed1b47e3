"""Write ``limit_gradients.json``: oracle gradients of one head at the block-count limit.

The attention kernels accept at most 16384 blocks per volume.  At that size the fp64
oracle needs minutes per head (every query block sees about 16,357 summaries), too long
for a GPU test, so this script runs it once on the CPU and stores the gradients of the
tokens of a few sampled blocks (corner, edge, interior and random ones; every token of
each block, so a row swapped or misplaced inside a block is caught).  It calls only the
oracle and the seeded input generator; the GPU test regenerates the same inputs and
compares its own gradients for those tokens with the stored values.

Run from the repository root:  python tests/golden/make_limit_gradients.py
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "limit_gradients.json")

# (name, dtype, heads, head_dim, head compared, sampled blocks): the two variants of the
# GPU limit test, 32x64x64 tokens in 2x2x2 blocks (16x32x32 = 16384 blocks), radius 1
CASES = [
    ("fp32_d12", torch.float32, 1, 12, 0, 16),
    ("bf16_d96", torch.bfloat16, 2, 96, 1, 5),
]
GRID, BLOCK, RADIUS, SEED = (32, 64, 64), (2, 2, 2), 1, 61


def sampled_blocks(nb, count, seed):
    """Corner, edge and interior blocks plus random ones (block ids, raster over the block grid)."""
    nbz, nby, nbx = nb
    ids = {0, nbz * nby * nbx - 1, nbx - 1, (nby - 1) * nbx, (nbz // 2 * nby + nby // 2) * nbx + nbx // 2,
           ((nbz - 1) * nby) * nbx + nbx // 2}
    rng = np.random.default_rng(seed)
    while len(ids) < count:
        ids.add(int(rng.integers(0, nbz * nby * nbx)))
    return sorted(ids)


def main():
    out = {"what": __doc__.split("\n\n")[1].replace("\n", " "),
           "grid": GRID, "block": BLOCK, "radius": RADIUS, "seed": SEED, "packing": "random",
           "generator": "synthetic_inputs.make_inputs(small_workload(...), dtype, with_grad=True); the gradients "
                        "are those of sum(o * dO) for the workload's dO plus 0.75 (the limit test's offset)",
           "cases": {}}
    nb = tuple(g // b for g, b in zip(GRID, BLOCK))
    for name, dtype, heads, d, head, nsample in CASES:
        t0 = time.time()
        w = si.small_workload(grid=GRID, block=BLOCK, radius=RADIUS, heads=heads, head_dim=d, packing="random",
                              seed=SEED)
        x = si.make_inputs(w, dtype, with_grad=True)
        x["do"] = (x["do"].float() + 0.75).to(dtype)
        one = {n: x[n][:, :, head:head + 1].contiguous() for n in ("q", "k", "v", "do")}
        ix = oracle.build_index(x["coords"].numpy(), BLOCK, RADIUS)[0]
        blocks = sampled_blocks(nb, nsample, SEED)
        tokens = [int(t) for b in blocks for t in ix["perm"][b * ix["bvol"]:(b + 1) * ix["bvol"]]]
        dq, dk, dv = oracle.backward(one["q"], one["k"], one["v"], x["coords"], one["do"], BLOCK, RADIUS)
        # significant digits: far below the tolerance of the dtype (1e-5 fp32, 2e-2 bf16)
        fmt = "{:.9e}" if dtype == torch.float32 else "{:.6e}"
        rows = lambda a: [[float(fmt.format(v)) for v in a[0, t, 0]] for t in tokens]
        out["cases"][name] = {"dtype": str(dtype).replace("torch.", ""), "heads": heads, "head_dim": d,
                              "head": head, "blocks": blocks, "tokens": tokens,
                              "dq": rows(dq), "dk": rows(dk), "dv": rows(dv)}
        print(f"{name}: {len(tokens)} tokens, {time.time() - t0:.0f} s", flush=True)
    with open(OUT, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
