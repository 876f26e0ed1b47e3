"""The forward entry point that allocates nothing (pack3d_forward_noalloc), through the C ABI,
against pack3d_forward with a caller workspace: bitwise equal outputs on two calls in a row,
the second with a smaller input, and refusal of a forward whose workspace exceeds the fixed
device buffer."""
import ctypes

import pytest
import torch

import synthetic_inputs as si
import sparse_local_global_amd.pack3d as p3
from tests.gpu_cases import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc_c(ix, attn, xd, out, lse):
    lib = p3.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    return lib.pack3d_forward_noalloc(ix.handle, ctypes.byref(attn), ptr(xd["q"]), ptr(xd["k"]), ptr(xd["v"]),
                                      ptr(xd["coords"]), ptr(out), ptr(lse),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


CALLS = [
    # the 16k workload (76 MB of workspace in bf16), then a much smaller one in fp32
    (si.WORKLOADS["16k"], torch.bfloat16),
    (si.small_workload(grid=(8, 8, 16), block=(4, 4, 4), heads=2, head_dim=48, packing="random", seed=81),
     torch.float32),
]


def test_forward_noalloc_matches_forward_twice():
    for w, dtype in CALLS:
        say(f"forward_noalloc {w.name} {dtype}")
        xd = to_dev(si.make_inputs(w, dtype))
        ix = p3.build_index(xd["coords"], w.block, w.radius)
        attn = p3.make_attn(dtype, w.heads, w.head_dim, w.rope_base)
        need = p3.workspace_bytes(ix, attn)
        assert 0 < need <= p3.NOALLOC_MAX_BYTES
        ref_o, ref_l = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base)
        out = torch.full_like(xd["q"], float("nan"))
        lse = torch.full((w.batch, w.heads, w.tokens), float("nan"), dtype=torch.float32, device=DEV)
        st = _noalloc_c(ix, attn, xd, out, lse)
        torch.cuda.synchronize()
        assert st == p3.OK, p3.load_library().pack3d_last_error()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        # and through the binding, windowed-only
        o2, l2 = p3.forward_noalloc(ix, xd["q"], xd["k"], xd["v"], xd["coords"], torch.empty_like(out),
                                    torch.empty_like(lse), rope_base=w.rope_base, with_summaries=False)
        r2, rl2 = p3.forward(ix, xd["q"], xd["k"], xd["v"], xd["coords"], rope_base=w.rope_base,
                             with_summaries=False)
        torch.cuda.synchronize()
        assert torch.equal(o2, r2) and torch.equal(l2, rl2)


def test_forward_noalloc_refuses_beyond_its_buffer():
    w = si.WORKLOADS["65k"]
    dtype = torch.bfloat16
    say("forward_noalloc beyond its buffer")
    xd = to_dev(si.make_inputs(w, dtype))
    ix = p3.build_index(xd["coords"], w.block, w.radius)
    attn = p3.make_attn(dtype, w.heads, w.head_dim, w.rope_base)
    assert p3.workspace_bytes(ix, attn) > p3.NOALLOC_MAX_BYTES
    out = torch.zeros_like(xd["q"])
    lse = torch.zeros((w.batch, w.heads, w.tokens), dtype=torch.float32, device=DEV)
    st = _noalloc_c(ix, attn, xd, out, lse)
    torch.cuda.synchronize()
    assert st == p3.E_WORKSPACE
    assert b"fixed device scratch buffer" in p3.load_library().pack3d_last_error()
    assert torch.count_nonzero(out) == 0 and torch.count_nonzero(lse) == 0
