"""A pre-norm transformer block around the PACK3D operator, for end-to-end training.

"Geometry Matters in Packed 3D Attention" (abstract): the operator is a trainable
attention layer for packed 3D data.  The block around it is the standard pre-norm layout
(the pages give none):

    x1 = x + W_o PACK3D(split(W_qkv LN1(x)))
    y  = x1 + W_2 GELU(W_1 LN2(x1))

The projections are plain matrix products (torch -> hipBLASLt); the QKV projection's output
[T, 3 C] is read by the library in place as [T, 3, H, D] (pack3d_forward_qkv), and its
gradient is written in place by pack3d_backward_qkv, so no split or concatenation copy sits
between the projection and the operator.  The attention output [T, H, D] is the output
projection's input as [T, C] without a copy.
"""
from __future__ import annotations

import torch

from .pack3d import Index, attention_qkv


class Pack3DBlock(torch.nn.Module):
    def __init__(self, dim: int, heads: int, mlp_ratio: int = 4, rope_base: float = 10000.0,
                 device=None, dtype=None, position_mode: str = "axial"):
        super().__init__()
        if dim % heads:
            raise ValueError("dim must be a multiple of heads")
        kw = dict(device=device, dtype=dtype)
        self.dim, self.heads, self.rope_base = dim, heads, rope_base
        self.position_mode = position_mode  # rotation of the operator (see pack3d.make_attn)
        self.norm1 = torch.nn.LayerNorm(dim, eps=1e-5, **kw)
        self.qkv = torch.nn.Linear(dim, 3 * dim, bias=False, **kw)
        self.proj = torch.nn.Linear(dim, dim, bias=False, **kw)
        self.norm2 = torch.nn.LayerNorm(dim, eps=1e-5, **kw)
        self.fc1 = torch.nn.Linear(dim, mlp_ratio * dim, bias=False, **kw)
        self.fc2 = torch.nn.Linear(mlp_ratio * dim, dim, bias=False, **kw)

    def load_params(self, params: dict):
        """Copy weights from a dict of tensors named ln1_w, ln1_b, qkv ([3C, C]), proj, ln2_w,
        ln2_b, fc1 ([mlp_ratio C, C]) and fc2, each in torch.nn.Linear / LayerNorm layout."""
        with torch.no_grad():
            for mod, name in ((self.norm1.weight, "ln1_w"), (self.norm1.bias, "ln1_b"), (self.qkv.weight, "qkv"),
                              (self.proj.weight, "proj"), (self.norm2.weight, "ln2_w"), (self.norm2.bias, "ln2_b"),
                              (self.fc1.weight, "fc1"), (self.fc2.weight, "fc2")):
                mod.copy_(params[name].to(mod.dtype))

    def forward(self, x: torch.Tensor, index: Index, coords: torch.Tensor) -> torch.Tensor:
        """x [T, C] or [B, N, C] in the index's packed order."""
        shape = x.shape
        x = x.reshape(-1, self.dim)
        t = x.shape[0]
        d = self.dim // self.heads
        qkv = self.qkv(self.norm1(x)).view(t, 3, self.heads, d)
        a = attention_qkv(qkv, index, coords, rope_base=self.rope_base, position_mode=self.position_mode)
        x1 = x + self.proj(a.view(t, self.dim))
        y = x1 + self.fc2(torch.nn.functional.gelu(self.fc1(self.norm2(x1))))
        return y.view(shape)
