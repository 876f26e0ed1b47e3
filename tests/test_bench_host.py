"""Host logic of bench.py (no GPU): the one-GPU refusal, the pair counts behind the flop
figures, and the source-hash gate on the stored HBM counters."""
import json

import numpy as np
import torch

import bench
import oracle


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_refused_under_a_multi_rank_launch(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2
    assert "WORLD_SIZE 4" in capsys.readouterr().err


def _axis_neighbours(n: int, r: int) -> int:
    """Sum over the n positions of an axis of the number of positions within distance r."""
    return sum(min(i + r, n - 1) - max(i - r, 0) + 1 for i in range(n))


def test_pair_counts_of_the_65k_geometry():
    """The flop figures rest on these counts: on a full block grid the local blocks of a block
    are a product of per-axis windows, so their total is a product of per-axis sums."""
    grid, block, r = (32, 32, 64), (4, 4, 4), 1
    z, y, x = np.meshgrid(*[np.arange(g) for g in grid], indexing="ij")
    coords = np.stack([z.ravel(), y.ravel(), x.ravel()], 1).astype(np.int64)
    ref = oracle.build_index(coords, block, r)[0]
    tables = {"nbr": torch.from_numpy(np.asarray(ref["nbr"])[None]), "block_tokens": 64, "nblk": ref["nblk"]}
    local, summ = bench.pair_counts(tables)
    nb = [g // b for g, b in zip(grid, block)]
    neighbours = np.prod([_axis_neighbours(n, r) for n in nb])
    nblk, bvol = int(np.prod(nb)), int(np.prod(block))
    assert local == neighbours * bvol * bvol == 91_193_344
    assert summ == (nblk * nblk - neighbours) * bvol == 65_683_968


def test_stored_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_local_global_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    rec = {"source_hash": h1, "kernels": {"bwd_dq": {"bytes_per_launch": 2.0e9}}}
    (tmp_path / "profiles" / "hbm_traffic_65k.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("bwd_dq") == 2.0e9
    assert bench.stored_traffic("attn_fwd") is None
    (csrc / "k.hip").write_text("// kernel v2\n")
    assert bench.kernel_source_hash() != h1
    assert bench.stored_traffic("bwd_dq") is None

