"""GPU backward (dq, dk, dv through the softmax, the block mean pooling and the RoPE)
against the fp64 oracle.  Tolerances: max-abs 1e-5 (fp32 inputs), 2e-2 (bf16 inputs,
fp32 accumulation)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.dense_ref import torch_axial_rope
from tests.gpu_cases import DEV, TOL, max_err, sample_blocks, say, to_dev
from tests.test_gpu_forward import CASES

pytestmark = pytest.mark.gpu


def gpu_backward(w, dtype, x=None, with_summaries=True, **kw):
    if x is None:
        x = si.make_inputs(w, dtype, with_grad=True, **kw)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base,
                          with_summaries=with_summaries)
    dq, dk, dv = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"],
                             rope_base=w.rope_base, with_summaries=with_summaries)
    torch.cuda.synchronize()
    return x, (dq, dk, dv)


@pytest.mark.parametrize("grid,block,r,heads,d,packing,batch,dtype", CASES)
@pytest.mark.parametrize("with_s", [True, False])
def test_backward_matches_oracle_small(grid, block, r, heads, d, packing, batch, dtype, with_s):
    w = si.small_workload(grid=grid, block=block, radius=r, heads=heads, head_dim=d, packing=packing,
                          batch=batch, seed=19)
    say(f"backward {grid} {block} r={r} H={heads} D={d} {packing} B={batch} {dtype} summaries={with_s}")
    x, grads = gpu_backward(w, dtype, with_summaries=with_s)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], block, r, with_summaries=with_s)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        err = max_err(g, rr)
        assert err < TOL[dtype], (name, err)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_16k_workload_full(dtype):
    w = si.WORKLOADS["16k"]
    say(f"backward 16k {dtype}")
    x, grads = gpu_backward(w, dtype)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        assert max_err(g, rr) < TOL[dtype], name


def test_backward_65k_training_workload_one_head():
    """Full-size training step launch; the oracle computes every gradient of one (volume, head)."""
    w = si.WORKLOADS["65k-train"]
    dtype = torch.bfloat16
    say("backward 65k training workload")
    x, grads = gpu_backward(w, dtype)
    vol, head = 1, 5
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius,
                          volumes=[vol], heads=[head])
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        gg = g[vol][:, head].float().cpu().double().numpy()
        assert np.abs(gg - rr[vol][:, head]).max() < TOL[dtype], name
        assert torch.isfinite(g).all(), name


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_256_token_blocks_with_summaries_full(dtype):
    """256-token blocks (4x8x8) on a 4x4x4 block grid, so at r = 1 every query has both
    local keys (up to 27 blocks of four 64-row tiles) and summaries: the multi-tile cursor
    paths of the key-major and summary-major backward kernels.  Forward and every gradient
    element by element against the oracle."""
    w = si.small_workload(grid=(16, 32, 32), block=(4, 8, 8), radius=1, heads=2, head_dim=96, packing="random",
                          seed=29)
    say(f"256-token blocks with summaries {dtype}")
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base)
    grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], rope_base=w.rope_base)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], x["coords"], w.block, w.radius)
    assert max_err(out, o_ref) < TOL[dtype] and max_err(lse, l_ref) < TOL[dtype]
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius)
    for name, g, rr in zip(("dq", "dk", "dv"), grads, ref):
        err = max_err(g, rr)
        say(f"  {name}: max err {err:.3e}")
        assert err < TOL[dtype], (name, err)


def test_backward_524k_sampled_dq_and_identities():
    """The 524k workload: one volume of 32x128x128 tokens in 256-token blocks (4x8x8), so each
    block is four 64-query tiles and a query sees up to 6,912 local keys and 2,025 summaries.
    dq of sampled query blocks against the oracle.  dk and dv need every query, so over all
    524,288 tokens they are held to two exact identities of the method (each query's weights
    over keys and summaries sum to one, and a block mean hands a summary's gradient to its
    members in full):
        sum_j dv_j = sum_i dO_i        and        sum_j R_j dk_j = 0
    per (head, channel), R_j the token's rotation.  Bound: 2^-7 of sum_i |dO_i| (bf16 products
    and bf16 gradients, as at the block-count limit)."""
    w = si.WORKLOADS["524k"]
    dtype = torch.bfloat16
    say("backward 524k")
    x = si.make_inputs(w, dtype, with_grad=True)
    x["do"] = (x["do"].float() + 0.75).to(dtype)   # a mean offset makes the dv identity sensitive
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base)
    dq, dk, dv = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"],
                             rope_base=w.rope_base)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    nb = tuple(g // b for g, b in zip(w.grid, w.block))
    blocks = sample_blocks(nb, count=6, seed=w.seed)
    dq_ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius,
                             query_blocks=blocks)[0]
    mask = ~np.isnan(dq_ref)
    assert mask.sum() == len(blocks) * int(np.prod(w.block)) * w.heads * w.head_dim
    assert max_err(dq, dq_ref, mask) < TOL[dtype]
    del dq_ref, mask
    do64 = xd["do"][0].double()
    scale = do64.abs().sum(0)                                            # [H, D]
    gap = dv[0].double().sum(0) - do64.sum(0)
    assert (gap.abs() <= 2.0 ** -7 * scale).all(), float((gap.abs() / scale).max())
    c = x["coords"][0].long()
    rot = torch_axial_rope(dk[0].double().cpu(), c - c.min(0).values, w.rope_base).sum(0)
    scale = scale.cpu()
    assert (rot.abs() <= 2.0 ** -7 * scale).all(), float((rot.abs() / scale).max())


def test_backward_deterministic_and_repacking_bitwise():
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, packing="random", seed=6)
    dtype = torch.bfloat16
    _, g1 = gpu_backward(w, dtype)
    _, g2 = gpu_backward(w, dtype)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    ref = None
    for packing in si.PACKINGS:
        x, g = gpu_backward(w, dtype, packing=packing)
        inv = torch.argsort(x["perm"][0]).to(DEV)
        g = [t[0][inv] for t in g]
        if ref is None:
            ref = g
        else:
            for a, b in zip(g, ref):
                assert torch.equal(a, b), packing
    _, g3 = gpu_backward(w, dtype, shift=(-9, 4, 77))
    for a, b in zip(g1, g3):
        assert torch.equal(a, b)


def test_autograd_wrapper():
    w = si.small_workload(grid=(8, 8, 8), block=(2, 2, 4), heads=2, head_dim=48, packing="morton", seed=12)
    dtype = torch.float32
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    q, k, v = (xd[n].clone().requires_grad_() for n in ("q", "k", "v"))
    coords = xd["coords"].clone()
    o = p3.attention(q, k, v, ix, coords)
    (o * xd["do"]).sum().backward(retain_graph=True)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["coords"], x["do"], w.block, w.radius)
    for g, rr in zip((q.grad, k.grad, v.grad), ref):
        assert max_err(g, rr) < TOL[dtype]
    # a second backward through the retained graph recomputes the freed intermediates:
    # the gradients accumulate to exactly twice the first ones
    first = [t.grad.clone() for t in (q, k, v)]
    (o * xd["do"]).sum().backward()
    for t, g in zip((q, k, v), first):
        assert torch.equal(t.grad, 2 * g)
    # coordinates changed in place after the forward are caught by autograd
    o = p3.attention(q, k, v, ix, coords)
    coords.add_(1)
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        (o * xd["do"]).sum().backward()


def test_backward_poisoned_workspace():
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=48, packing="random", seed=8)
    dtype = torch.float32
    x, g1 = gpu_backward(w, dtype)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"])
    attn = p3.make_attn(dtype, w.heads, w.head_dim)
    ws = torch.full((p3.workspace_bytes(ix, attn, True) // 4,), float("nan"), device=DEV).view(torch.uint8)
    g2 = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_reusing_forward_workspace_bitwise(dtype):
    """reuse_forward skips recomputing the forward's intermediates; gradients are bitwise equal."""
    w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, packing="random", seed=21)
    say(f"backward reuse {dtype}")
    xd = to_dev(si.make_inputs(w, dtype, with_grad=True))
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    attn = p3.make_attn(dtype, w.heads, w.head_dim)
    ws = torch.full((p3.workspace_bytes(ix, attn, True),), 255, dtype=torch.uint8, device=DEV)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], workspace=ws)
    ref = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"])
    got = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], workspace=ws,
                      reuse_forward=True)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    with pytest.raises(p3.Pack3DError):
        p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], reuse_forward=True)


def test_backward_errors():
    """Caller buffers of the wrong dtype or size, and gradient pointers that are not 16-byte
    aligned, are refused before any launch."""
    w = si.small_workload(grid=(4, 4, 8), block=(2, 2, 2), heads=1, head_dim=12, seed=1)
    x = to_dev(si.make_inputs(w, torch.float32, with_grad=True))
    ix = p3.build_index(x["coords"], w.block, 1)
    out, lse = p3.forward(ix, x["q"], x["k"], x["v"], x["coords"])
    attn = p3.make_attn(torch.float32, 1, 12)
    ws = torch.empty(p3.workspace_bytes(ix, attn, True), dtype=torch.uint8, device=DEV)
    args = (ix, x["q"], x["k"], x["v"], x["coords"], out)
    for lse_bad in (lse.double(), lse[:, :, :-1]):
        with pytest.raises(p3.Pack3DError) as e:
            p3.backward(*args, lse_bad, x["do"])
        assert e.value.status == p3.E_INVALID
    with pytest.raises(p3.Pack3DError) as e:
        p3.backward(*args, lse, x["do"], workspace=ws.view(torch.float32))
    assert e.value.status == p3.E_INVALID
    # C ABI with dq one element off 16-byte alignment (the buffer has room for that offset)
    lib = p3.load_library()
    g = torch.zeros(3 * w.tokens * 12 + 8, device=DEV)
    base = g.data_ptr()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    dq = ctypes.c_void_p(base + 4)
    dk = ctypes.c_void_p(base + 4 * (w.tokens * 12 + 4))
    dv = ctypes.c_void_p(base + 4 * (2 * w.tokens * 12 + 8))
    st = lib.pack3d_backward(ix.handle, ctypes.byref(attn), ptr(x["q"]), ptr(x["k"]), ptr(x["v"]), ptr(x["coords"]),
                             ptr(out), ptr(lse), ptr(x["do"]), dq, dk, dv, ptr(ws), ws.numel(), 0, None)
    torch.cuda.synchronize()
    assert st == p3.E_INVALID and b"16-byte aligned" in lib.pack3d_last_error()
    assert torch.count_nonzero(g) == 0


@pytest.mark.timeout(900)
def test_backward_524k_one_head_elementwise():
    """The 524k workload at full size (the launch the benchmark would make): every
    gradient of one head, element by element, against the oracle.  Heads are independent,
    so the oracle runs on that head's slice of q, k, v and dO."""
    w = si.WORKLOADS["524k"]
    dtype = torch.bfloat16
    head = 6
    say("backward 524k, one head element-wise")
    x = si.make_inputs(w, dtype, with_grad=True)
    xd = to_dev(x)
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    out, lse = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base)
    grads = p3.backward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], out, lse, xd["do"], rope_base=w.rope_base)
    torch.cuda.synchronize()
    got = [g[:, :, head:head + 1].float().cpu().double().numpy() for g in grads]
    del xd, out, lse, grads
    one = {n: x[n][:, :, head:head + 1].contiguous() for n in ("q", "k", "v", "do")}
    say("  oracle backward of one head")
    ref = oracle.backward(one["q"], one["k"], one["v"], x["coords"], one["do"], w.block, w.radius)
    for name, g, rr in zip(("dq", "dk", "dv"), got, ref):
        err = float(np.abs(g - rr).max())
        say(f"  {name}: max err {err:.3e}")
        assert err < TOL[dtype], (name, err)
