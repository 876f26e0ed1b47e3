#!/usr/bin/env python
"""PACK3D benchmark on one MI355X: tokens/s and ms per step at 65,536 tokens per volume.

Workload: 2 volumes of 32x32x64 = 65,536 tokens (131,072 per call), random
packing, 8 heads, head dim 96, 4x4x4 blocks (1,024 per volume), local radius 1
(3x3x3 blocks), bf16 with fp32 accumulation, synthetic N(0,1) inputs.

A step is one pass of the hot path over that batch with the index already built
(it depends on the geometry only and is built once, timed separately): the forward
(RoPE/gather/pooling, fused attention) and, when the library provides it, the
backward, which reuses the rotated and pooled operands the forward left in its
workspace (as the autograd wrapper does).  Inputs are resident in HBM before the
timed region starts.

Printed: one JSON line with the contract fields, the roofline of the dominant
kernel (the matrix-core kernel with the most time per step: bwd_dq in the training
step, the fused attention forward in a forward-only run) from HIP events recorded by
the library around each launch on its stream, every kernel's rate, the windowed-only
(local keys only) latency of the attention forward, and the fp64 CPU oracle timed on
a bounded sample (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PACK3D fwd(+bwd) tokens/s and ms at 65k tokens; MFMA util % of peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the HIP sources, tying a stored counter measurement to the code it measured."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_local_global_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when the summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_65k.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def pair_counts(tables: dict) -> tuple[int, int]:
    """(local pairs, summary pairs) per (volume, head), from the neighbour table of volume 0."""
    nbr = tables["nbr"][0].cpu()
    bvol, nblk = tables["block_tokens"], tables["nblk"]
    nloc = (nbr >= 0).sum(1).long()
    local = int((nloc * bvol * bvol).sum())
    summ = int(((nblk - nloc) * bvol).sum())
    return local, summ


def time_region(fn, steps: int):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


def gemm_ceiling(steps: int = 20, n: int = 8192) -> dict:
    """Attainable bf16 matrix-core rate on this GPU: a square torch.matmul (hipBLASLt), timed
    after the step timings, as a reference beside the datasheet peak."""
    import torch
    a = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    ms = time_region(lambda: torch.matmul(a, b), steps)
    del a, b
    return {"tflops": 2.0 * n ** 3 / (ms * 1e-3) / 1e12, "shape_mnk": [n, n, n], "ms": ms,
            "library": "torch.matmul (hipBLASLt), bf16 in, fp32 accumulate"}


def ragged_step(name: str, steps: int, warmup: int) -> dict:
    """Forward + backward step on a ragged varlen batch (partial edge blocks, holes, two volume
    shapes), timed like the headline step; per-kernel averages from the library's events."""
    import torch
    import synthetic_inputs as si
    import sparse_local_global_amd.pack3d as p3
    spec = si.RAGGED_WORKLOADS[name]
    x = si.make_ragged_inputs(spec["grids"], spec["heads"], spec["head_dim"], torch.bfloat16,
                              occupancy=spec["occupancy"], seed=spec["seed"], with_grad=True)
    off = x["offsets"].tolist()
    xd = {k: v.to("cuda:0") for k, v in x.items() if k in ("q", "k", "v", "coords", "do")}
    ix = p3.build_index(xd["coords"], spec["block"], spec["radius"], ragged=True, offsets=off)
    attn = p3.make_attn(torch.bfloat16, spec["heads"], spec["head_dim"])
    ws = torch.empty(p3.workspace_bytes(ix, attn, True), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(xd["q"])
    lse = torch.empty((ix.batch, spec["heads"], ix.tokens), dtype=torch.float32, device="cuda:0")

    def step():
        p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], workspace=ws, out=out, lse=lse)
        p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], workspace=ws,
                    reuse_forward=True)

    for _ in range(warmup):
        step()
    ms = time_region(step, steps)
    p3.profile_reset()
    p3.profile_enable(True)
    time_region(step, steps)
    prof = p3.profile_read()
    p3.profile_enable(False)
    t = ix.tables()
    tokens = off[-1]
    return {"workload": name, "description": spec["description"], "tokens": tokens,
            "canonical_slots": ix.batch * t["nblk"] * t["block_tokens"], "ms_per_step": ms,
            "tokens_per_s": tokens / (ms * 1e-3), "pass": "forward+backward",
            "kernels_avg_ms": {k: tt / max(n, 1) for k, (n, tt) in prof.items()}}


def block_step(w, coords, steps: int, warmup: int) -> dict:
    """Training step of one pre-norm transformer block around the operator at the workload's
    shapes (C = H * D, MLP 4 C, bf16, random init): forward, then backward for the input and
    every weight.  The projections are hipBLASLt GEMMs through torch; the operator runs from
    the QKV projection's output in place."""
    import torch
    import sparse_local_global_amd.pack3d as p3
    from sparse_local_global_amd.block import Pack3DBlock
    c = w.heads * w.head_dim
    torch.manual_seed(0)
    m = Pack3DBlock(c, w.heads, rope_base=w.rope_base, device="cuda:0", dtype=torch.bfloat16)
    x = torch.randn((w.batch, w.tokens, c), device="cuda:0", dtype=torch.bfloat16).requires_grad_()
    dy = torch.randn_like(x)
    ix = p3.build_index(coords, w.block, w.radius, order_hint=w.packing)

    def step():
        m.zero_grad(set_to_none=True)
        x.grad = None
        (m(x, ix, coords) * dy).sum().backward()

    for _ in range(warmup):
        step()
    ms = time_region(step, steps)
    p3.profile_reset()
    p3.profile_enable(True)
    time_region(step, steps)
    prof = p3.profile_read()
    p3.profile_enable(False)
    op_ms = sum(t for _, t in prof.values()) / steps
    tokens = w.batch * w.tokens
    gemm_flop = 3 * 2.0 * tokens * c * (3 * c + c + 2 * 4 * c)   # forward + two backward products each
    return {"model": f"pre-norm block, C={c}, heads={w.heads}, MLP 4C, bf16", "tokens": tokens,
            "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3), "operator_ms_per_step": op_ms,
            "operator_share": op_ms / ms, "gemm_flop_per_step": gemm_flop,
            "other_tflops": gemm_flop / ((ms - op_ms) * 1e-3) / 1e12}


def cpu_baseline(w, x, sample_blocks: int) -> dict:
    """The fp64 oracle on the host cores, in the metric's unit (tokens/s of a forward + backward
    step), from two bounded samples of the same workload: the forward of all heads of the first
    `sample_blocks` query blocks of each volume, and the backward (every gradient) of volume 0,
    head 0.  Each sample gives a token rate for all heads; the step rate combines the two."""
    import oracle  # test infrastructure, used only for this reported baseline
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # threadpoolctl missing: numpy's BLAS uses every core
        cores = os.cpu_count() or 1
    bvol = int(w.block[0] * w.block[1] * w.block[2])
    blocks = list(range(sample_blocks))
    t0 = time.perf_counter()
    oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius, query_blocks=blocks)
    dt_f = time.perf_counter() - t0
    fwd_tokens = w.batch * sample_blocks * bvol
    fwd_rate = fwd_tokens / dt_f
    t0 = time.perf_counter()
    oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius, volumes=[0], heads=[0])
    dt_b = time.perf_counter() - t0
    bwd_rate = w.tokens / w.heads / dt_b   # one head of one volume: 1/H of that volume's token work
    step_rate = 1.0 / (1.0 / fwd_rate + 1.0 / bwd_rate)
    return {"value": step_rate, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"forward: {sample_blocks} of {w.tokens // bvol} query blocks per volume, all {w.heads} "
                      f"heads, both volumes ({fwd_tokens} query tokens, {dt_f:.1f} s including the whole-volume "
                      f"RoPE and pooling); backward: every gradient of volume 0, head 0 of {w.heads} "
                      f"({w.tokens} tokens, {dt_b:.1f} s); value = 1 / (1 / forward rate + 1 / backward rate), "
                      f"fp64 NumPy",
            "forward_tokens_per_s": fwd_rate, "backward_tokens_per_s": bwd_rate}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="65k")
    ap.add_argument("--forward-only", action="store_true", help="time the forward alone")
    ap.add_argument("--position-mode", default="axial", choices=["axial", "packed1d", "none"],
                    help="rotation of the timed step (axial grid-coordinate RoPE is the method)")
    ap.add_argument("--no-mode-compare", action="store_true",
                    help="skip timing the step under the other position modes")
    ap.add_argument("--no-block", action="store_true",
                    help="skip timing the transformer-block training step around the operator")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip timing the step on the ragged varlen stand-in (partial blocks, holes)")
    ap.add_argument("--cpu-sample-blocks", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-ceiling", action="store_true", help="skip the hipBLASLt GEMM reference")
    ap.add_argument("--profile-pass", choices=["step", "forward", "windowed", "gemm"], default=None,
                    help="only run warmup + steps of one pass (the step, the forward, the windowed-only "
                         "forward, or the hipBLASLt reference GEMM) and print its time: for profiler runs, so "
                         "each pass has its own rows")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for HBM counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); the operator "
              f"is benchmarked per GPU and the library has no multi-GPU path.", file=sys.stderr)
        return 2

    import torch
    if args.profile_pass == "gemm":
        # the hipBLASLt reference GEMM alone, for the matrix-core counters of a plain GEMM
        ms = gemm_ceiling(args.steps)["ms"]
        print(json.dumps({"profile_pass": "gemm", "ms": ms, "steps": args.steps}))
        return 0
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return 0
    import synthetic_inputs as si
    import sparse_local_global_amd.pack3d as p3

    w = si.WORKLOADS[args.workload]
    dtype = torch.bfloat16
    log(f"bench: generating {w.description}")
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = {k: v.to("cuda:0") for k, v in x.items()}
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    ix = p3.build_index(xd["coords"], w.block, w.radius, order_hint=w.packing)
    index_ms = (time.perf_counter() - t0) * 1000.0
    mode = args.position_mode
    ws_bytes = max(p3.workspace_bytes(ix, p3.make_attn(dtype, w.heads, w.head_dim, w.rope_base, position_mode=m),
                                      True) for m in p3.POSITION_MODES)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(xd["q"])
    lse = torch.empty((w.batch, w.heads, w.tokens), dtype=torch.float32, device="cuda:0")

    # a profiler pass over the forward alone launches no backward kernel at all
    with_bwd = not args.forward_only and args.profile_pass not in ("forward", "windowed")
    if with_bwd:
        try:
            p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], workspace=ws,
                        position_mode=mode)
        except p3.Pack3DError as e:
            if e.status != p3.E_UNSUPPORTED:
                raise
            log(f"bench: backward not available ({e}); timing the forward only")
            with_bwd = False

    def fwd(with_summaries=True, pm=None):
        p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], with_summaries=with_summaries,
                   workspace=ws, out=out, lse=lse, position_mode=pm or mode)

    def step(pm=None):
        fwd(pm=pm)
        if with_bwd:
            p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], workspace=ws,
                        reuse_forward=True, position_mode=pm or mode)

    if args.profile_pass:
        fn = {"step": step, "forward": fwd, "windowed": lambda: fwd(False)}[args.profile_pass]
        for _ in range(args.warmup):
            fn()
        ms = time_region(fn, args.steps)
        print(json.dumps({"profile_pass": args.profile_pass, "ms": ms, "steps": args.steps,
                          "warmup": args.warmup, "workload": args.workload,
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return 0

    for _ in range(args.warmup):
        step()
    log(f"bench: warmup done ({args.warmup} steps), timing {args.steps} steps")
    ms_step = time_region(step, args.steps)
    # the same steps timed one by one with events on the launch stream (median beside the mean)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    ms_step_median = per_step[len(per_step) // 2]

    # same steps again with per-kernel HIP events (library-side, on the launch stream)
    p3.profile_reset()
    p3.profile_enable(True)
    ms_step_profiled = time_region(step, args.steps)
    prof = p3.profile_read()
    p3.profile_enable(False)

    # windowed-only baseline: the same kernel with the summary stream off
    for _ in range(args.warmup):
        fwd(False)
    ms_fwd = time_region(fwd, args.steps)
    ms_win = time_region(lambda: fwd(False), args.steps)
    p3.profile_reset()
    p3.profile_enable(True)
    time_region(lambda: fwd(False), args.steps)
    prof_win = p3.profile_read()
    p3.profile_enable(False)
    log(f"bench: step {ms_step:.3f} ms, forward {ms_fwd:.3f} ms, windowed-only forward {ms_win:.3f} ms")

    # the same step under the other rotations (controls of the operator): whole step and rope_pool
    modes = {}
    if not args.no_mode_compare:
        for pm in p3.POSITION_MODES:
            for _ in range(args.warmup):
                step(pm)
            ms = time_region(lambda: step(pm), args.steps)
            p3.profile_reset()
            p3.profile_enable(True)
            time_region(lambda: step(pm), args.steps)
            pp = p3.profile_read()
            p3.profile_enable(False)
            modes[pm] = {"ms_per_step": ms, "tokens_per_s": w.batch * w.tokens / (ms * 1e-3),
                         "kernels_avg_ms": {k: t / max(n, 1) for k, (n, t) in pp.items()}}
            log(f"bench: position mode {pm}: step {ms:.3f} ms")

    local, summ = pair_counts(ix.tables())
    bh = w.batch * w.heads
    d = w.head_dim
    act = float(w.batch * w.tokens * w.heads * d * 2)          # one bf16 activation tensor
    # algorithmic work per launch: (flop or bytes, bound)
    work = {
        "attn_fwd": (4.0 * d * (local + summ) * bh, "mfma"),
        "attn_fwd_windowed": (4.0 * d * local * bh, "mfma"),
        "bwd_summary": (8.0 * d * summ * bh, "mfma"),      # S, dP, dVbar, dKbar per summary pair
        "bwd_local": (8.0 * d * local * bh, "mfma"),       # S, dP, dV, dK per local pair
        "bwd_dq": (2.0 * d * (local + summ) * bh, "mfma"), # dQ only: S and dP are recomputed
        "rope_pool": (6.0 * act, "hbm"),                    # read q, k, v; write Q~, K~, V canonical
        "rope_pool_bwd": (6.0 * act, "hbm"),                # recomputation (backward without reuse)
        "bwd_pre": (3.0 * act, "hbm"),                      # read dO, O; write dO canonical
    }
    # matrix-core work the kernel executes where it exceeds the algorithmic count (reported
    # beside it, never as the numerator): bwd_dq recomputes S and dP for its dQ product
    executed = {"bwd_dq": 6.0 * d * (local + summ) * bh}
    kern = {}
    for name, (n, t) in prof.items():
        avg = t / max(n, 1)
        entry = {"launches": n, "avg_ms": avg, "total_ms_per_step": t / args.steps}
        if name in work:
            amount, bound = work[name]
            rate = amount / (avg * 1e-3)
            if bound == "mfma":
                entry.update(bound="mfma", flop_per_launch=amount, tflops=rate / 1e12,
                             frac=rate / 1e12 / PEAK_BF16_TFLOPS)
                if name in executed:
                    erate = executed[name] / (avg * 1e-3) / 1e12
                    entry.update(executed_flop_per_launch=executed[name], executed_tflops=erate,
                                 executed_frac=erate / PEAK_BF16_TFLOPS)
            else:
                entry.update(bound="hbm", bytes_per_launch=amount, gbs=rate / 1e9, frac=rate / 1e9 / PEAK_HBM_GBS)
        kern[name] = entry
    dominant = max((k for k in kern if kern[k].get("bound") == "mfma"), key=lambda k: kern[k]["total_ms_per_step"])
    dk = kern[dominant]
    attn_ms = kern["attn_fwd"]["avg_ms"]
    win_attn_ms = prof_win["attn_fwd_windowed"][1] / max(prof_win["attn_fwd_windowed"][0], 1)
    fwd_flop = work["attn_fwd"][0]

    tokens = w.batch * w.tokens
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "65k", "pass": "forward+backward" if with_bwd else "forward",
                   "batch": w.batch, "grid_zyx": list(w.grid), "tokens_per_volume": w.tokens,
                   "tokens_per_step": tokens, "heads": w.heads, "head_dim": d, "block_zyx": list(w.block),
                   "local_radius": w.radius, "packing": w.packing, "position_mode": mode,
                   "accumulation": "fp32"},
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": dk["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": dk["frac"], "traffic": stored_traffic(dominant),
                     "flop_per_launch": dk["flop_per_launch"], "avg_launch_ms": dk["avg_ms"],
                     **({"executed_frac": dk["executed_frac"]} if "executed_frac" in dk else {})},
        "kernels": kern,
        "forward_ms": ms_fwd,
        "forward_tokens_per_s": tokens / (ms_fwd * 1e-3),
        "attn_fwd_tflops": fwd_flop / (attn_ms * 1e-3) / 1e12,
        "attn_fwd_mfma_frac": fwd_flop / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "windowed_forward_ms": ms_win,
        "forward_vs_windowed": ms_fwd / ms_win,
        "attn_vs_windowed_attn": attn_ms / win_attn_ms,
        "windowed_attn": {"avg_ms": win_attn_ms, "tflops": work["attn_fwd_windowed"][0] / (win_attn_ms * 1e-3) / 1e12},
        "index_build_ms": index_ms,
        "ms_per_step_with_kernel_events": ms_step_profiled,
        "ms_per_step_median_of_events": ms_step_median,
        "pairs_per_volume_head": {"local": local, "summary": summ},
        "kernel_source_hash": kernel_source_hash(),
    }
    if modes:
        result["position_modes"] = modes
    if not args.no_block and with_bwd:
        blk = block_step(w, xd["coords"], args.steps, args.warmup)
        log(f"bench: transformer block step {blk['ms_per_step']:.3f} ms (operator {blk['operator_ms_per_step']:.3f} ms)")
        result["block"] = blk
    if not args.no_ragged and with_bwd:
        rg = ragged_step("65k-ragged", args.steps, args.warmup)
        log(f"bench: ragged 65k-ragged: step {rg['ms_per_step']:.3f} ms ({rg['tokens']} tokens)")
        result["ragged"] = rg
    if not args.no_gemm_ceiling:
        g = gemm_ceiling()
        result["gemm_ceiling"] = g
        result["roofline"]["frac_of_gemm_ceiling"] = dk["tflops"] / g["tflops"]
        result["attn_fwd_frac_of_gemm_ceiling"] = result["attn_fwd_tflops"] / g["tflops"]
    if not args.no_cpu_baseline:
        log(f"bench: timing the fp64 oracle (forward sample of {args.cpu_sample_blocks} query blocks per "
            f"volume, backward of one volume and head)")
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_sample_blocks)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
