"""GPU fused-projection entry points and the PACK3D transformer block against the fp64 oracle.

The fused entry points read q, k, v from one [T, 3, H, D] buffer and write the gradients into
one such buffer; they must equal the separate-tensor entry points bitwise.  The block
(sparse_local_global_amd.block) is compared with oracle/block.py on the same weights
(rounded to the tested dtype), output and every gradient.
Tolerances (max-abs error over the largest reference magnitude of the tensor): fp32 1e-4;
bf16 3e-2.  Derivation: fp32 runs about ten dependent steps whose products sum at most
4 C = 768 terms, so accumulated rounding stays well below 1e-5 relative, and the operator's
own fp32 bar is 1e-5; the margin covers the GEMM library's summation order.  In bf16 every
stored activation is rounded to 8 significant bits (relative 2^-9 = 2e-3), about eight
roundings lie on any path (LayerNorm, QKV, operator, projection, residual, LayerNorm, MLP,
residual), and the operator alone is held to 2e-2 of unit-scale outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.block as ob
import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from sparse_local_global_amd.block import Pack3DBlock
from tests.gpu_cases import DEV, say

pytestmark = pytest.mark.gpu

BLOCK_TOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}


def _rel_err(gpu, ref):
    g = gpu.detach().double().cpu().numpy()
    r = ref.detach().double().cpu().numpy() if torch.is_tensor(ref) else ref
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("ragged", [False, True])
def test_fused_entry_points_bitwise_equal_separate(dtype, ragged):
    say(f"fused qkv {dtype} ragged={ragged}")
    g = torch.Generator().manual_seed(5)
    if ragged:
        x = si.make_ragged_inputs([(9, 10, 13), (7, 8, 9)], 2, 96, dtype, occupancy=0.8, seed=91)
        coords, off = x["coords"].to(DEV), x["offsets"].tolist()
        ix = p3.build_index(coords, (4, 4, 4), 1, ragged=True, offsets=off)
        t = off[-1]
    else:
        w = si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=96, batch=2, seed=92)
        xi = si.make_inputs(w, dtype)
        coords = xi["coords"].to(DEV)
        ix = p3.build_index(coords, w.block, w.radius)
        t = w.batch * w.tokens
    qkv = torch.randn((t, 3, 2, 96), generator=g).to(dtype).to(DEV)
    dout = torch.randn((t, 2, 96), generator=g).to(dtype).to(DEV)
    out, lse = p3.forward_qkv(ix, qkv, coords)
    dqkv = p3.backward_qkv(ix, qkv, coords, out, lse, dout)
    q, k, v = (qkv[:, s].contiguous() for s in range(3))
    shape = ix.act_shape(2, 96)
    q, k, v = (a.view(shape) for a in (q, k, v))
    out2, lse2 = p3.forward(ix, q, k, v, coords)
    dq, dk, dv = p3.backward(ix, q, k, v, coords, out2, lse2, dout.view(shape))
    torch.cuda.synchronize()
    assert torch.equal(out.view(shape), out2)
    counts = np.diff(off) if ragged else [w.tokens] * w.batch
    for vol, n in enumerate(counts):      # lse past a volume's token count is not written
        assert torch.equal(lse[vol, :, :n], lse2[vol, :, :n]), vol
    for s, gsep in enumerate((dq, dk, dv)):
        assert torch.equal(dqkv[:, s].reshape(shape), gsep), s


def _block_case(dtype, grid=(8, 8, 16), block=(4, 4, 4), heads=2, d=96, batch=2, seed=93):
    w = si.small_workload(grid=grid, block=block, heads=heads, head_dim=d, batch=batch, packing="random", seed=seed)
    coords = si.make_inputs(w, torch.float32)["coords"]
    c = heads * d
    gen = np.random.default_rng(seed + 7)
    x = torch.from_numpy(gen.standard_normal((batch, w.tokens, c))).to(dtype)
    dy = torch.from_numpy(gen.standard_normal((batch, w.tokens, c))).to(dtype)
    params = {k: v.to(dtype).double() for k, v in ob.init_params(c, seed=seed).items()}  # the dtype's weights
    return w, coords, x, dy, params


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_forward_backward_match_oracle(dtype):
    say(f"block {dtype}")
    w, coords, x, dy, params = _block_case(dtype)
    m = Pack3DBlock(w.heads * w.head_dim, w.heads, device=DEV, dtype=dtype)
    m.load_params(params)
    cd = coords.to(DEV)
    ix = p3.build_index(cd, w.block, w.radius)
    xd = x.to(DEV).requires_grad_()
    y = m(xd, ix, cd)
    (y * dy.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    xr = x.double().clone().requires_grad_()
    pr = {k: v.clone().requires_grad_() for k, v in params.items()}
    yr = ob.block_forward(xr, pr, coords.numpy(), w.block, w.radius, w.heads)
    (yr * dy.double()).sum().backward()
    errs = {"y": _rel_err(y, yr), "dx": _rel_err(xd.grad, xr.grad)}
    for name, mod in (("ln1_w", m.norm1.weight), ("ln1_b", m.norm1.bias), ("qkv", m.qkv.weight),
                      ("proj", m.proj.weight), ("ln2_w", m.norm2.weight), ("ln2_b", m.norm2.bias),
                      ("fc1", m.fc1.weight), ("fc2", m.fc2.weight)):
        errs[name] = _rel_err(mod.grad, pr[name].grad)
    say("  relative errors: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v < BLOCK_TOL[dtype], (k, v)


def test_block_autograd_fused_gradient_layout():
    """The autograd wrapper hands back dqkv in the fused layout: a finite-direction check of
    the attention step alone, against the separate-tensor backward."""
    w, coords, _, _, _ = _block_case(torch.float32, batch=1, seed=94)
    cd = coords.to(DEV)
    ix = p3.build_index(cd, w.block, w.radius)
    g = torch.Generator().manual_seed(9)
    qkv = torch.randn((w.tokens, 3, w.heads, w.head_dim), generator=g).to(DEV).requires_grad_()
    dout = torch.randn((w.tokens, w.heads, w.head_dim), generator=g).to(DEV)
    o = p3.attention_qkv(qkv, ix, cd)
    (o * dout).sum().backward()
    x = {"q": qkv[:, 0].detach().cpu()[None], "k": qkv[:, 1].detach().cpu()[None], "v": qkv[:, 2].detach().cpu()[None]}
    ref = oracle.backward(x["q"], x["k"], x["v"], coords, dout.cpu()[None], w.block, w.radius)
    for s in range(3):
        assert np.abs(qkv.grad[:, s].double().cpu().numpy() - ref[s][0]).max() < 1e-5, s


def test_block_65k_forward_sampled():
    """The block at the 65k shapes (2 x 65,536 tokens, C = 768, bf16): outputs of sampled
    query blocks against the oracle block (projections of every token in fp64, the operator
    on the sampled query blocks only)."""
    w = si.WORKLOADS["65k"]
    dtype = torch.bfloat16
    say("block 65k forward")
    c = w.heads * w.head_dim
    coords = si.make_inputs(si.small_workload(grid=w.grid, block=w.block, heads=1, head_dim=6, batch=w.batch,
                                              packing=w.packing, seed=w.seed), torch.float32)["coords"]
    gen = np.random.default_rng(95)
    x = torch.from_numpy(gen.standard_normal((w.batch, w.tokens, c), dtype=np.float32)).to(dtype)
    params = {k: v.to(dtype).double() for k, v in ob.init_params(c, seed=95).items()}
    m = Pack3DBlock(c, w.heads, device=DEV, dtype=dtype)
    m.load_params(params)
    cd = coords.to(DEV)
    ix = p3.build_index(cd, w.block, w.radius)
    with torch.no_grad():
        y = m(x.to(DEV), ix, cd).double().cpu()
    torch.cuda.synchronize()
    nb = tuple(g // b for g, b in zip(w.grid, w.block))
    from tests.gpu_cases import sample_blocks
    blocks = sample_blocks(nb, count=6, seed=w.seed)
    xr = x.double()
    with torch.no_grad():
        qkv = ob.layer_norm(xr, params["ln1_w"], params["ln1_b"]) @ params["qkv"].T
        q, k, v = (qkv[..., s * c:(s + 1) * c].reshape(w.batch, w.tokens, w.heads, w.head_dim) for s in range(3))
        o, _ = oracle.forward(q.numpy(), k.numpy(), v.numpy(), coords.numpy(), w.block, w.radius,
                              query_blocks=blocks)
        rows = ~np.isnan(o[..., 0, 0])                       # [B, N] sampled tokens
        a = torch.from_numpy(o[rows].reshape(-1, c))
        x1 = xr[torch.from_numpy(rows)] + a @ params["proj"].T
        yr = x1 + ob.gelu(ob.layer_norm(x1, params["ln2_w"], params["ln2_b"]) @ params["fc1"].T) @ params["fc2"].T
    err = _rel_err(y[torch.from_numpy(rows)], yr)
    say(f"  65k block: {int(rows.sum())} sampled tokens, relative error {err:.2e}")
    assert err < BLOCK_TOL[dtype]
