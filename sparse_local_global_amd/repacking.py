"""Synthetic repacking experiment: train on one packing, evaluate on others.

"Geometry Matters in Packed 3D Attention" (abstract) measures the failure mode of
position encodings indexed by the packed sequence on a controlled synthetic task: a
model is trained on one packing of the tokens, then only the memory order of the tokens
changes while the physical labeling rule stays the same.  Encodings tied to the packed
position fit the training layout and fail under Morton, block-contiguous and random
repacking; axial RoPE on the true grid coordinates is unaffected.

The pages give neither the task nor its labeling rule.  Reading used here (the plainest
geometry-only rule; every choice below is this module's, not the pages'):

* A volume is a Z x Y x X grid.  Each voxel holds a class c in {0 .. K-1}, drawn uniformly
  and independently.  A token carries only the embedding of its own class.
* The label of the voxel at (z, y, x) is the pattern of its three forward neighbours,
      c(z + 1, y, x) + K c(z, y + 1, x) + K^2 c(z, y, x + 1)     (K^3 labels),
  a fixed function of its 3D neighbourhood computed from coordinates.  Voxels on the high
  faces (a neighbour missing) carry no label and count in neither loss nor accuracy.
  A model can only solve the task by locating its three neighbours, and each neighbour it
  finds pays off on its own (a rule that mixes them, such as their sum mod K, gives no
  training signal until all three are found).
* The model: class embedding -> L pre-norm blocks whose attention is PACK3D (radius 1
  around 2 x 2 x 2 blocks, so the three neighbours are always local keys) -> LayerNorm ->
  linear classifier.  Position mechanisms, all with the same operator (locality and
  summaries always follow the grid):
    axial     the method: axial RoPE on grid coordinates;
    packed1d  control: 1D RoPE on the packed position;
    learned   control: a learned embedding per packed position added to the input, no
              rotation;
    none      control: no position information (chance level, 1/K^3).
* Training: fresh random volumes every step (no example is seen twice), raster packing,
  AdamW, cross-entropy over labelled voxels, until the training layout is fitted (mean
  training accuracy 0.995 over 50 steps) or a budget of 12,000 steps is spent.  Evaluation: fresh volumes under raster,
  Morton, block-contiguous and random packings (the physical volume and its labels are
  the same; only the order of the tokens changes).

Run ``python -m sparse_local_global_amd.repacking`` for the full table (one GPU).
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from dataclasses import asdict, dataclass

import numpy as np
import torch

from . import pack3d as p3
from .block import Pack3DBlock

PACKINGS = ("raster", "morton", "block", "random")
POSITION_MECHANISMS = ("axial", "packed1d", "learned", "none")


@dataclass(frozen=True)
class TaskConfig:
    grid: tuple = (8, 8, 8)         # (Z, Y, X)
    classes: int = 2                # K: classes per voxel; K^3 labels
    block: tuple = (2, 2, 2)
    radius: int = 1
    heads: int = 4
    head_dim: int = 48
    layers: int = 2
    batch: int = 32                 # volumes per training step
    steps: int = 12000              # at most; training stops once the layout is fitted
    fit_accuracy: float = 0.995     # mean training accuracy over `fit_window` steps that stops it
    fit_window: int = 50
    lr: float = 1e-3
    pos_init: float = 1.0           # std of the learned position embeddings at initialisation
    eval_volumes: int = 16
    seed: int = 0

    @property
    def tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def labels(self) -> int:
        return self.classes ** 3


# ---- the labeling rule ------------------------------------------------------------------

def labels_from_grid(cls: torch.Tensor, classes: int) -> torch.Tensor:
    """cls [..., Z, Y, X] int64 -> labels [..., Z, Y, X]: c(z+1) + K c(y+1) + K^2 c(x+1), and -1
    on the high faces where a neighbour is missing."""
    lab = torch.full_like(cls, -1)
    core = cls[..., 1:, :-1, :-1] + classes * cls[..., :-1, 1:, :-1] + classes * classes * cls[..., :-1, :-1, 1:]
    lab[..., :-1, :-1, :-1] = core
    return lab


def raster_coords(grid) -> np.ndarray:
    z, y, x = grid
    zz, yy, xx = np.meshgrid(np.arange(z), np.arange(y), np.arange(x), indexing="ij")
    return np.stack([zz.ravel(), yy.ravel(), xx.ravel()], axis=1).astype(np.int32)


def morton_order(grid) -> np.ndarray:
    """Raster indices sorted by the 3D bit-interleaved code (x at bit 3k, y at 3k+1, z at 3k+2)."""
    c = raster_coords(grid).astype(np.uint64)
    code = np.zeros(c.shape[0], dtype=np.uint64)
    for bit in range(21):
        for axis, shift in ((2, 0), (1, 1), (0, 2)):
            code |= ((c[:, axis] >> np.uint64(bit)) & np.uint64(1)) << np.uint64(3 * bit + shift)
    return np.argsort(code, kind="stable")


def block_order(grid, block) -> np.ndarray:
    """Raster indices visited block by block (blocks in raster order, raster inside each)."""
    z, y, x = grid
    bz, by, bx = block
    idx = np.arange(z * y * x).reshape(z // bz, bz, y // by, by, x // bx, bx)
    return idx.transpose(0, 2, 4, 1, 3, 5).reshape(-1)


def packing_order(grid, packing: str, block, rng: np.random.Generator) -> np.ndarray:
    """perm[p] = raster index of the token stored at packed position p."""
    n = int(np.prod(grid))
    if packing == "raster":
        return np.arange(n)
    if packing == "morton":
        return morton_order(grid)
    if packing == "block":
        return block_order(grid, block)
    if packing == "random":
        return rng.permutation(n)
    raise ValueError(f"unknown packing {packing!r}")


def make_batch(cfg: TaskConfig, rng: np.random.Generator, packing: str, volumes: int, device):
    """Fresh volumes in one packing: classes and labels [B, N] (packed order), coords [B, N, 3]
    int32 and the packing permutations [B, N] (packed position -> raster index)."""
    z, y, x = cfg.grid
    cls = torch.from_numpy(rng.integers(0, cfg.classes, size=(volumes, z, y, x)))
    lab = labels_from_grid(cls, cfg.classes)
    rc = torch.from_numpy(raster_coords(cfg.grid))
    perms = torch.from_numpy(np.stack([packing_order(cfg.grid, packing, cfg.block, rng) for _ in range(volumes)]))
    cls_p = torch.stack([cls[v].reshape(-1)[perms[v]] for v in range(volumes)])
    lab_p = torch.stack([lab[v].reshape(-1)[perms[v]] for v in range(volumes)])
    coords = torch.stack([rc[perms[v]] for v in range(volumes)]).contiguous()
    return cls_p.to(device), lab_p.to(device), coords.to(device), perms


# ---- the model ----------------------------------------------------------------------------

class RepackModel(torch.nn.Module):
    """Class embedding -> PACK3D blocks -> LayerNorm -> classifier, with one position mechanism."""

    def __init__(self, cfg: TaskConfig, mechanism: str, device, dtype=torch.float32):
        super().__init__()
        if mechanism not in POSITION_MECHANISMS:
            raise ValueError(f"mechanism must be one of {POSITION_MECHANISMS}")
        c = cfg.heads * cfg.head_dim
        kw = dict(device=device, dtype=dtype)
        self.cfg, self.mechanism = cfg, mechanism
        self.embed = torch.nn.Embedding(cfg.classes, c, **kw)
        self.pos = (torch.nn.Parameter(cfg.pos_init * torch.randn(cfg.tokens, c, **kw))
                    if mechanism == "learned" else None)
        mode = mechanism if mechanism in ("axial", "packed1d") else "none"
        self.blocks = torch.nn.ModuleList(
            [Pack3DBlock(c, cfg.heads, device=device, dtype=dtype, position_mode=mode) for _ in range(cfg.layers)])
        self.norm = torch.nn.LayerNorm(c, **kw)
        self.head = torch.nn.Linear(c, cfg.labels, **kw)

    def forward(self, cls: torch.Tensor, index: p3.Index, coords: torch.Tensor) -> torch.Tensor:
        """cls [B, N] in packed order -> logits [B, N, K^3]."""
        h = self.embed(cls)
        if self.pos is not None:
            h = h + self.pos      # indexed by packed position: the layout, not the geometry
        for blk in self.blocks:
            h = blk(h, index, coords)
        return self.head(self.norm(h))


def _accuracy(logits, lab):
    keep = lab >= 0
    return float((logits.argmax(-1)[keep] == lab[keep]).float().mean())


def train(cfg: TaskConfig, mechanism: str, device="cuda:0", log=None):
    """Train on raster-packed volumes until the training layout is fitted (mean accuracy over
    the last ``fit_window`` steps at least ``fit_accuracy``) or ``steps`` steps; returns the
    model and the number of steps taken.  The learning rate warms up over 200 steps and then
    stays constant."""
    torch.manual_seed(cfg.seed)
    rng = np.random.default_rng(cfg.seed)
    model = RepackModel(cfg, mechanism, device)
    opt = torch.optim.AdamW(model.parameters(), lr=cfg.lr, weight_decay=0.01)
    sched = torch.optim.lr_scheduler.LambdaLR(opt, lambda s: min(1.0, (s + 1) / 200))
    index = None
    recent = []
    step = 0
    for step in range(cfg.steps):
        cls, lab, coords, _ = make_batch(cfg, rng, "raster", cfg.batch, device)
        if index is None:   # raster coordinates are the same every step
            index = p3.build_index(coords, cfg.block, cfg.radius, order_hint="raster")
        logits = model(cls, index, coords)
        keep = lab >= 0
        loss = torch.nn.functional.cross_entropy(logits[keep], lab[keep])
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        sched.step()
        recent = (recent + [_accuracy(logits, lab)])[-cfg.fit_window:]
        if log is not None and step % 500 == 0:
            log(f"{mechanism} step {step}: loss {float(loss):.4f} accuracy {recent[-1]:.4f}")
        if len(recent) == cfg.fit_window and sum(recent) / len(recent) >= cfg.fit_accuracy:
            break
    if log is not None:
        log(f"{mechanism}: stopped after {step + 1} steps, training accuracy {sum(recent) / len(recent):.4f}")
    return model, step + 1


@torch.no_grad()
def evaluate(model: RepackModel, cfg: TaskConfig, packing: str, device="cuda:0", seed: int = 12345):
    """Accuracy on fresh volumes packed as ``packing``, plus the predictions in raster order
    [V, N] (so two packings of the same volumes can be compared token by token)."""
    rng = np.random.default_rng(seed)
    z, y, x = cfg.grid
    cls = torch.from_numpy(rng.integers(0, cfg.classes, size=(cfg.eval_volumes, z, y, x)))
    lab = labels_from_grid(cls, cfg.classes)
    prng = np.random.default_rng(seed + 1)
    perms = torch.from_numpy(np.stack([packing_order(cfg.grid, packing, cfg.block, prng)
                                       for _ in range(cfg.eval_volumes)]))
    rc = torch.from_numpy(raster_coords(cfg.grid))
    cls_p = torch.stack([cls[v].reshape(-1)[perms[v]] for v in range(cfg.eval_volumes)]).to(device)
    lab_p = torch.stack([lab[v].reshape(-1)[perms[v]] for v in range(cfg.eval_volumes)]).to(device)
    coords = torch.stack([rc[perms[v]] for v in range(cfg.eval_volumes)]).contiguous().to(device)
    index = p3.build_index(coords, cfg.block, cfg.radius, order_hint=packing)
    logits = model(cls_p, index, coords)
    pred = logits.argmax(-1).cpu()
    raster_pred = torch.empty_like(pred)
    for v in range(cfg.eval_volumes):
        raster_pred[v, perms[v]] = pred[v]
    return _accuracy(logits, lab_p), raster_pred, logits


def run(cfg: TaskConfig, mechanisms=POSITION_MECHANISMS, device="cuda:0", log=print) -> dict:
    """Train one model per mechanism on raster packing; accuracy under every packing."""
    table = {}
    for mech in mechanisms:
        t0 = time.perf_counter()
        model, steps = train(cfg, mech, device, log)
        train_s = time.perf_counter() - t0
        row = {}
        preds = {}
        for packing in PACKINGS:
            acc, pred, _ = evaluate(model, cfg, packing, device)
            row[packing] = acc
            preds[packing] = pred
        # fraction of voxels whose prediction is unchanged by repacking (raster order compared)
        row["same_prediction_as_raster"] = {pk: float((preds[pk] == preds["raster"]).float().mean())
                                            for pk in PACKINGS if pk != "raster"}
        row["train_steps"] = steps
        row["train_seconds"] = train_s
        table[mech] = row
        log(f"{mech}: " + ", ".join(f"{pk} {row[pk]:.4f}" for pk in PACKINGS) + f" ({train_s:.0f} s)")
    return {"config": asdict(cfg), "chance": 1.0 / cfg.labels, "accuracy": table}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="train on raster packing, evaluate under repacking")
    ap.add_argument("--steps", type=int, default=TaskConfig.steps)
    ap.add_argument("--layers", type=int, default=TaskConfig.layers)
    ap.add_argument("--seed", type=int, default=TaskConfig.seed)
    ap.add_argument("--lr", type=float, default=TaskConfig.lr)
    ap.add_argument("--pos-init", type=float, default=TaskConfig.pos_init)
    ap.add_argument("--mechanisms", default=",".join(POSITION_MECHANISMS))
    args = ap.parse_args(argv)
    cfg = TaskConfig(steps=args.steps, layers=args.layers, seed=args.seed, lr=args.lr, pos_init=args.pos_init)
    res = run(cfg, tuple(args.mechanisms.split(",")), log=lambda *a: print(*a, file=sys.stderr, flush=True))
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
