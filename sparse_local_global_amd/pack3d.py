"""Python binding of libpack3d (the PACK3D C ABI declared in include/pack3d.h).

Argument marshalling only: torch supplies device memory and the stream, every
step of the operator runs in the library's HIP kernels.  If the library is not
built, or is loaded without a GPU, calls raise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpack3d.so")

OK, E_INVALID, E_COORDS, E_UNSUPPORTED, E_WORKSPACE, E_HIP = range(6)
F32, BF16 = 0, 1
ORDERS = {"any": 0, "raster": 1, "morton": 2, "block": 3, "random": 4}
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class Pack3DError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pack3d status {status}: {message}")
        self.status = status


class Packing(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("tokens_per_volume", ctypes.c_int32), ("order_hint", ctypes.c_int32),
                ("ragged", ctypes.c_int32), ("volume_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("max_blocks", ctypes.c_int32)]


class Attn(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("with_summaries", ctypes.c_int32), ("position_mode", ctypes.c_int32)]


class Tables(ctypes.Structure):
    _fields_ = [("token_block", ctypes.c_void_p), ("canon", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("nbr", ctypes.c_void_p), ("geom", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("tokens", ctypes.c_int32), ("nblk", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("slots", ctypes.c_int32), ("radius", ctypes.c_int32),
                ("block_shape", ctypes.c_int32 * 3), ("extent_max", ctypes.c_int32 * 3),
                ("block_count", ctypes.c_void_p), ("volume_offsets", ctypes.c_void_p),
                ("total_tokens", ctypes.c_int64), ("ragged", ctypes.c_int32), ("holes", ctypes.c_int32)]


GEOM_FIELDS = 10


class Views(ctypes.Structure):
    _fields_ = [("rope_table", ctypes.c_size_t), ("qrot", ctypes.c_size_t), ("krot", ctypes.c_size_t),
                ("vrow", ctypes.c_size_t), ("kbar", ctypes.c_size_t), ("vbar", ctypes.c_size_t),
                ("head_dim_padded", ctypes.c_int32), ("nblk_padded", ctypes.c_int32),
                ("extent_table", ctypes.c_int32)]


EXPORTS = {
    "pack3d_index_bytes": (ctypes.c_size_t, [ctypes.POINTER(Packing), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]),
    "pack3d_build_index": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Packing), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_void_p)]),
    "pack3d_measure_blocks": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Packing), ctypes.POINTER(ctypes.c_int32),
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.POINTER(ctypes.c_int32)]),
    "pack3d_index_tables": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Tables)]),
    "pack3d_index_geometry": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "pack3d_index_free": (None, [ctypes.c_void_p]),
    "pack3d_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.POINTER(Attn), ctypes.c_int]),
    "pack3d_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn)] + [ctypes.c_void_p] * 6
                       + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pack3d_backward": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn)] + [ctypes.c_void_p] * 10
                        + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]),
    "pack3d_forward_qkv": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn)] + [ctypes.c_void_p] * 4
                           + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "pack3d_backward_qkv": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn)] + [ctypes.c_void_p] * 6
                            + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]),
    "pack3d_forward_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn)] + [ctypes.c_void_p] * 6
                               + [ctypes.c_void_p]),
    "pack3d_workspace_views": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Attn), ctypes.POINTER(Views)]),
    "pack3d_profile_enable": (ctypes.c_int, [ctypes.c_int32]),
    "pack3d_profile_read": (ctypes.c_int32, [ctypes.c_char_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_double), ctypes.c_int32]),
    "pack3d_profile_reset": (None, []),
    "pack3d_last_error": (ctypes.c_char_p, []),
    "pack3d_version": (ctypes.c_int32, []),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpack3d.so (after torch, so the process holds a single HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise Pack3DError(E_INVALID, f"{path} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != OK:
        raise Pack3DError(status, load_library().pack3d_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Index:
    """A built PACK3D index: the device tables (owned here) plus the library handle.

    ``offsets`` is None for the uniform layout ([B, N, ...] tensors) or the B + 1 token
    offsets of a varlen batch (flat [T, ...] tensors); ``tokens`` is the largest volume."""

    def __init__(self, handle, tables: torch.Tensor, batch, tokens, block_shape, radius, offsets=None,
                 ragged=False):
        self._handle = handle
        self.tables_buffer = tables
        self.batch, self.tokens = batch, tokens
        self.block_shape, self.radius = tuple(block_shape), radius
        self.offsets = None if offsets is None else [int(o) for o in offsets]
        self.total = batch * tokens if offsets is None else self.offsets[-1]
        self.ragged = ragged

    @property
    def device(self) -> torch.device:
        """The GPU holding the index's tables; every tensor used with the index must be on it."""
        return self.tables_buffer.device

    def act_shape(self, h, d):
        """Shape of q, k, v, out and the gradients for this layout."""
        return (self.batch, self.tokens, h, d) if self.offsets is None else (self.total, h, d)

    @property
    def handle(self):
        if self._handle is None:
            raise Pack3DError(E_INVALID, "index has been freed")
        return self._handle

    def free(self):
        if self._handle is not None:
            load_library().pack3d_index_free(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def _view(self, ptr, count):
        base = self.tables_buffer.data_ptr()
        off = ptr - base
        return self.tables_buffer[off: off + 4 * count].view(torch.int32)

    def tables(self) -> dict:
        """Device views: token_block, canon [B, N] (uniform) or [T] (varlen); perm [B, nblk |b|]
        (-1 = empty slot); nbr [B, nblk, slots]; block_count [B, nblk]; geom [B, 10]."""
        t = Tables()
        _check(load_library().pack3d_index_tables(self.handle, ctypes.byref(t)))
        b, nblk, slots, total = t.batch, t.nblk, t.slots, t.total_tokens
        tok_shape = (b, t.tokens) if self.offsets is None else (total,)
        nc = nblk * t.block_tokens
        return dict(token_block=self._view(t.token_block, total).view(*tok_shape),
                    canon=self._view(t.canon, total).view(*tok_shape),
                    perm=self._view(t.perm, b * nc).view(b, nc),
                    nbr=self._view(t.nbr, b * nblk * slots).view(b, nblk, slots),
                    block_count=self._view(t.block_count, b * nblk).view(b, nblk),
                    volume_offsets=self._view(t.volume_offsets, b + 1),
                    geom=self._view(t.geom, b * GEOM_FIELDS).view(b, GEOM_FIELDS),
                    nblk=nblk, block_tokens=t.block_tokens, slots=slots,
                    extent_max=tuple(t.extent_max), ragged=bool(t.ragged), holes=bool(t.holes))

    def geometry(self, volume: int):
        out = (ctypes.c_int32 * 6)()
        _check(load_library().pack3d_index_geometry(self.handle, volume, out))
        return tuple(out[:3]), tuple(out[3:])


def _packing(batch, tokens, order_hint="any", ragged=False, offsets=None, max_blocks=0):
    """Packing struct; the offsets array is kept alive on the struct."""
    p = Packing(batch, tokens, ORDERS.get(order_hint, 0), 1 if ragged else 0, None, max_blocks)
    if offsets is not None:
        arr = (ctypes.c_int32 * len(offsets))(*[int(o) for o in offsets])
        p.volume_offsets = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        p._keep = arr
    return p


def index_bytes(batch, tokens, block_shape, radius, *, ragged=False, offsets=None, max_blocks=0) -> int:
    p = _packing(batch, tokens, ragged=ragged, offsets=offsets, max_blocks=max_blocks)
    bs = (ctypes.c_int32 * 3)(*block_shape)
    return load_library().pack3d_index_bytes(ctypes.byref(p), bs, radius)


def measure_blocks(coords: torch.Tensor, block_shape, *, offsets=None) -> int:
    """Blocks per volume (the largest) that ragged coordinates need (synchronizes)."""
    lib = load_library()
    b, n = _coords_layout(coords, offsets)
    p = _packing(b, n, ragged=True, offsets=offsets)
    bs = (ctypes.c_int32 * 3)(*block_shape)
    scratch = torch.empty(64 * b, dtype=torch.uint8, device=coords.device)
    out = ctypes.c_int32()
    with torch.cuda.device(coords.device):
        _check(lib.pack3d_measure_blocks(_ptr(coords.contiguous()), ctypes.byref(p), bs, _ptr(scratch),
                                         scratch.numel(), ctypes.c_void_p(_stream()), ctypes.byref(out)))
    return out.value


def _coords_layout(coords, offsets):
    """(batch, tokens per volume or 0) of coords [B, N, 3] or flat [T, 3] with offsets."""
    if coords.dtype != torch.int32 or coords.shape[-1] != 3 or not coords.is_cuda:
        raise Pack3DError(E_INVALID, "coords must be a CUDA int32 tensor [B, N, 3] or [T, 3]")
    if offsets is None:
        if coords.dim() != 3:
            raise Pack3DError(E_INVALID, "coords must be [B, N, 3] without offsets")
        return coords.shape[0], coords.shape[1]
    if coords.dim() != 2 or int(offsets[-1]) != coords.shape[0]:
        raise Pack3DError(E_INVALID, "with offsets, coords must be [T, 3] with T = offsets[-1]")
    return len(offsets) - 1, 0


def build_index(coords: torch.Tensor, block_shape, local_radius: int, order_hint: str = "any", *,
                ragged: bool = False, offsets=None) -> Index:
    """coords: int32 [B, N, 3] (z, y, x) on the GPU, or flat [T, 3] with ``offsets`` (B + 1 host
    ints) for volumes of different token counts.  ``ragged``: any set of distinct points
    (partial edge blocks, holes); otherwise every volume must be a full grid divisible by the
    block."""
    lib = load_library()
    b, n = _coords_layout(coords, offsets)
    coords = coords.contiguous()
    max_blocks = measure_blocks(coords, block_shape, offsets=offsets) if ragged else 0
    p = _packing(b, n, order_hint, ragged, offsets, max_blocks)
    bs = (ctypes.c_int32 * 3)(*block_shape)
    nbytes = lib.pack3d_index_bytes(ctypes.byref(p), bs, local_radius)
    if nbytes == 0:
        raise Pack3DError(E_INVALID, "invalid batch layout, block shape or radius")
    tables = torch.empty(nbytes, dtype=torch.uint8, device=coords.device)
    handle = ctypes.c_void_p()
    with torch.cuda.device(coords.device):
        _check(lib.pack3d_build_index(_ptr(coords), ctypes.byref(p), bs, local_radius, _ptr(tables),
                                      nbytes, ctypes.c_void_p(_stream()), ctypes.byref(handle)))
    nmax = n if offsets is None else max(int(offsets[i + 1]) - int(offsets[i]) for i in range(b))
    return Index(handle, tables, b, nmax, block_shape, local_radius, offsets, ragged)


POSITION_MODES = {"axial": 0, "packed1d": 1, "none": 2}


def make_attn(dtype, heads, head_dim, rope_base=10000.0, scale=None, with_summaries=True,
              position_mode="axial") -> Attn:
    """position_mode: "axial" (grid-coordinate RoPE, the method), "packed1d" (1D RoPE on the
    packed position) or "none" (no rotation); the last two are controls."""
    if dtype not in _DTYPES:
        raise Pack3DError(E_UNSUPPORTED, f"dtype {dtype} is not supported")
    if position_mode not in POSITION_MODES:
        raise Pack3DError(E_INVALID, f"position_mode {position_mode!r} is not one of {sorted(POSITION_MODES)}")
    return Attn(_DTYPES[dtype], heads, head_dim, float(rope_base), 0.0 if scale is None else float(scale),
                1 if with_summaries else 0, POSITION_MODES[position_mode])


def workspace_bytes(index: Index, attn: Attn, for_backward: bool = False) -> int:
    return load_library().pack3d_workspace_bytes(index.handle, ctypes.byref(attn), 1 if for_backward else 0)


def _check_act(name, t, shape, dtype):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda or not t.is_contiguous():
        raise Pack3DError(E_INVALID, f"{name} must be a contiguous CUDA {dtype} tensor of shape {tuple(shape)}")


# The library reads and writes these buffers at the sizes the index and the head count imply,
# so every one a caller hands in is checked against them here.
def _check_coords(index: Index, coords):
    want = index.act_shape(1, 3)[:-2] + (3,)
    if coords.dtype != torch.int32 or not coords.is_cuda or tuple(coords.shape) != tuple(want):
        raise Pack3DError(E_INVALID, f"coords must be the index's CUDA int32 coordinates of shape {want}")


def _check_lse(index: Index, lse, h):
    want = (index.batch, h, index.tokens)
    if lse.dtype != torch.float32 or not lse.is_cuda or tuple(lse.shape) != want or not lse.is_contiguous():
        raise Pack3DError(E_INVALID, f"lse must be a contiguous CUDA float32 tensor of shape {want}")


def _check_device(index: Index, *tensors):
    for t in tensors:
        if t is not None and t.device != index.device:
            raise Pack3DError(E_INVALID, f"tensors must be on the index's device {index.device}, not {t.device}")


def _check_workspace(ws):
    # its byte count is passed as the workspace size
    if ws.dtype != torch.uint8 or not ws.is_cuda or not ws.is_contiguous():
        raise Pack3DError(E_INVALID, "workspace must be a contiguous CUDA uint8 tensor")


def forward(index: Index, q, k, v, coords, *, rope_base=10000.0, scale=None, with_summaries=True,
            workspace: torch.Tensor | None = None, out=None, lse=None, position_mode="axial"):
    """PACK3D forward.  q, k, v [B, N, H, D] (or [T, H, D] for a varlen index); returns (out
    shaped like q, lse fp32 [B, H, Nmax])."""
    lib = load_library()
    h, d = q.shape[-2], q.shape[-1]
    b, n = index.batch, index.tokens
    attn = make_attn(q.dtype, h, d, rope_base, scale, with_summaries, position_mode)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_act(name, t, index.act_shape(h, d), q.dtype)
    _check_coords(index, coords)
    need = workspace_bytes(index, attn)
    if need == 0:
        raise Pack3DError(E_UNSUPPORTED, lib.pack3d_last_error().decode())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    if out is None:
        out = torch.empty_like(q)
    _check_act("out", out, index.act_shape(h, d), q.dtype)
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    _check_lse(index, lse, h)
    _check_device(index, q, k, v, coords, workspace, out, lse)
    with torch.cuda.device(index.device):
        _check(lib.pack3d_forward(index.handle, ctypes.byref(attn), _ptr(q), _ptr(k), _ptr(v), _ptr(coords.contiguous()),
                                  _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  ctypes.c_void_p(_stream())))
    return out, lse


def forward_noalloc(index: Index, q, k, v, coords, out, lse, *, rope_base=10000.0, scale=None,
                    with_summaries=True, position_mode="axial"):
    """The forward for callers that cannot allocate: the library's fixed device buffer is the
    workspace (at most NOALLOC_MAX_BYTES) and the caller passes ``out`` and ``lse``; results
    are bitwise those of ``forward``.  Calls that overlap on one GPU race on that buffer."""
    lib = load_library()
    h, d = q.shape[-2], q.shape[-1]
    attn = make_attn(q.dtype, h, d, rope_base, scale, with_summaries, position_mode)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_act(name, t, index.act_shape(h, d), q.dtype)
    _check_coords(index, coords)
    _check_lse(index, lse, h)
    _check_device(index, q, k, v, coords, out, lse)
    with torch.cuda.device(index.device):
        _check(lib.pack3d_forward_noalloc(index.handle, ctypes.byref(attn), _ptr(q), _ptr(k), _ptr(v), _ptr(coords),
                                          _ptr(out), _ptr(lse), ctypes.c_void_p(_stream())))
    return out, lse


NOALLOC_MAX_BYTES = 128 << 20   # PACK3D_NOALLOC_MAX_BYTES of include/pack3d.h


def backward(index: Index, q, k, v, coords, out, lse, dout, *, rope_base=10000.0, scale=None,
             with_summaries=True, workspace: torch.Tensor | None = None, reuse_forward: bool = False,
             position_mode="axial"):
    """Gradients (dq, dk, dv) of sum(out * dout) with respect to the unrotated q, k, v.

    reuse_forward=True: ``workspace`` is the one the forward of these inputs used (allocated
    with workspace_bytes(..., for_backward=True)) and still holds its intermediates, so the
    backward skips recomputing them."""
    lib = load_library()
    h, d = q.shape[-2], q.shape[-1]
    attn = make_attn(q.dtype, h, d, rope_base, scale, with_summaries, position_mode)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_act(name, t, index.act_shape(h, d), q.dtype)
    _check_coords(index, coords)
    lse = lse.contiguous()
    _check_lse(index, lse, h)
    need = workspace_bytes(index, attn, True)
    if need == 0:
        raise Pack3DError(E_UNSUPPORTED, lib.pack3d_last_error().decode())
    if workspace is None:
        if reuse_forward:
            raise Pack3DError(E_INVALID, "reuse_forward needs the forward's workspace")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check_device(index, q, k, v, coords, out, lse, dout, workspace)
    with torch.cuda.device(index.device):
        _check(lib.pack3d_backward(index.handle, ctypes.byref(attn), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(coords.contiguous()), _ptr(out), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                   1 if reuse_forward else 0, ctypes.c_void_p(_stream())))
    return dq, dk, dv


def forward_qkv(index: Index, qkv, coords, *, rope_base=10000.0, scale=None, with_summaries=True,
                workspace: torch.Tensor | None = None, out=None, lse=None, position_mode="axial"):
    """PACK3D forward from one fused projection output qkv [T, 3, H, D] (q, k, v = qkv[:, 0],
    qkv[:, 1], qkv[:, 2]; T = every token of the batch).  Returns (out [T, H, D], lse fp32
    [B, H, Nmax])."""
    lib = load_library()
    t, three, h, d = qkv.shape
    if three != 3 or t != index.total:
        raise Pack3DError(E_INVALID, f"qkv must be [{index.total}, 3, H, D]")
    attn = make_attn(qkv.dtype, h, d, rope_base, scale, with_summaries, position_mode)
    _check_act("qkv", qkv, (t, 3, h, d), qkv.dtype)
    _check_coords(index, coords)
    need = workspace_bytes(index, attn)
    if need == 0:
        raise Pack3DError(E_UNSUPPORTED, lib.pack3d_last_error().decode())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qkv.device)
    _check_workspace(workspace)
    if out is None:
        out = torch.empty((t, h, d), dtype=qkv.dtype, device=qkv.device)
    _check_act("out", out, (t, h, d), qkv.dtype)
    if lse is None:
        lse = torch.empty((index.batch, h, index.tokens), dtype=torch.float32, device=qkv.device)
    _check_lse(index, lse, h)
    _check_device(index, qkv, coords, workspace, out, lse)
    with torch.cuda.device(index.device):
        _check(lib.pack3d_forward_qkv(index.handle, ctypes.byref(attn), _ptr(qkv), _ptr(coords.contiguous()),
                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                      ctypes.c_void_p(_stream())))
    return out, lse


def backward_qkv(index: Index, qkv, coords, out, lse, dout, *, rope_base=10000.0, scale=None,
                 with_summaries=True, workspace: torch.Tensor | None = None, reuse_forward: bool = False,
                 position_mode="axial"):
    """Gradient dqkv [T, 3, H, D] of sum(out * dout) with respect to the fused qkv input."""
    lib = load_library()
    t, _, h, d = qkv.shape
    attn = make_attn(qkv.dtype, h, d, rope_base, scale, with_summaries, position_mode)
    _check_act("qkv", qkv, (index.total, 3, h, d), qkv.dtype)
    for name, x in (("out", out), ("dout", dout)):
        _check_act(name, x, (index.total, h, d), qkv.dtype)
    _check_coords(index, coords)
    lse = lse.contiguous()
    _check_lse(index, lse, h)
    need = workspace_bytes(index, attn, True)
    if need == 0:
        raise Pack3DError(E_UNSUPPORTED, lib.pack3d_last_error().decode())
    if workspace is None:
        if reuse_forward:
            raise Pack3DError(E_INVALID, "reuse_forward needs the forward's workspace")
        workspace = torch.empty(need, dtype=torch.uint8, device=qkv.device)
    _check_workspace(workspace)
    dqkv = torch.empty_like(qkv)
    _check_device(index, qkv, coords, out, lse, dout, workspace)
    with torch.cuda.device(index.device):
        _check(lib.pack3d_backward_qkv(index.handle, ctypes.byref(attn), _ptr(qkv), _ptr(coords.contiguous()), _ptr(out),
                                       _ptr(lse), _ptr(dout), _ptr(dqkv), _ptr(workspace),
                                       workspace.numel(), 1 if reuse_forward else 0, ctypes.c_void_p(_stream())))
    return dqkv


def workspace_views(index: Index, q_shape, dtype, workspace: torch.Tensor, rope_base=10000.0,
                    position_mode="axial") -> dict:
    """Tensor views of the forward intermediates left in ``workspace`` (canonical rows:
    nblk * |b| per volume)."""
    h, d = q_shape[-2], q_shape[-1]
    b = index.batch
    attn = make_attn(dtype, h, d, rope_base, position_mode=position_mode)
    vw = Views()
    _check(load_library().pack3d_workspace_views(index.handle, ctypes.byref(attn), ctypes.byref(vw)))
    t = index.tables()
    n = t["nblk"] * t["block_tokens"]
    dp, nbp = vw.head_dim_padded, vw.nblk_padded
    es = 2 if dtype == torch.bfloat16 else 4

    def view(off, shape, dt=dtype, esize=es):
        cnt = math.prod(shape)
        return workspace[off: off + cnt * esize].view(dt).view(*shape)

    half = d // 6 if position_mode == "axial" else d // 2     # pairs per rotation group
    return dict(rope_table=view(vw.rope_table, (vw.extent_table, half, 2), torch.float32, 4),
                qrot=view(vw.qrot, (b, h, n, dp)), krot=view(vw.krot, (b, h, n, dp)),
                vrow=view(vw.vrow, (b, h, n, dp)), kbar=view(vw.kbar, (b, h, nbp, dp)),
                vbar=view(vw.vbar, (b, h, nbp, dp)))


def profile_enable(enable: bool = True):
    """Bracket every library kernel launch with HIP events on its stream (see profile_read)."""
    _check(load_library().pack3d_profile_enable(1 if enable else 0))


def profile_reset():
    load_library().pack3d_profile_reset()


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} since the last reset (waits for the events)."""
    n_max = 32
    names = ctypes.create_string_buffer(48 * n_max)
    launches = (ctypes.c_int32 * n_max)()
    ms = (ctypes.c_double * n_max)()
    n = load_library().pack3d_profile_read(names, len(names), launches, ms, n_max)
    if n < 0:
        raise Pack3DError(E_HIP, "profile_read: HIP event error")
    out, parts = {}, names.raw.split(b"\0")
    for i in range(n):
        out[parts[i].decode()] = (launches[i], ms[i])
    return out


class Pack3DAttention(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libpack3d."""

    @staticmethod
    def forward(ctx, q, k, v, index: Index, coords, rope_base=10000.0, scale=None, with_summaries=True,
                position_mode="axial"):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        # the workspace is sized for the backward and kept, so the backward reuses the
        # forward's rotated and pooled operands instead of recomputing them
        attn = make_attn(q.dtype, q.shape[-2], q.shape[-1], rope_base, scale, with_summaries, position_mode)
        need = workspace_bytes(index, attn, True)
        if need == 0:
            raise Pack3DError(E_UNSUPPORTED, load_library().pack3d_last_error().decode())
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        out, lse = forward(index, q, k, v, coords, rope_base=rope_base, scale=scale,
                           with_summaries=with_summaries, workspace=ws, position_mode=position_mode)
        # coords go through autograd's saved tensors too, so changing them in place before
        # the backward is an error rather than gradients for other coordinates
        ctx.save_for_backward(q, k, v, out, lse, coords)
        ctx.index, ctx.workspace = index, ws
        ctx.opts = (rope_base, scale, with_summaries, position_mode)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, coords = ctx.saved_tensors
        rope_base, scale, with_summaries, position_mode = ctx.opts
        # the first backward reuses the forward's intermediates and frees them; a second
        # one (retain_graph) recomputes them
        ws, ctx.workspace = ctx.workspace, None
        dq, dk, dv = backward(ctx.index, q, k, v, coords, out, lse, dout.contiguous(), rope_base=rope_base,
                              scale=scale, with_summaries=with_summaries, workspace=ws,
                              reuse_forward=ws is not None, position_mode=position_mode)
        return dq, dk, dv, None, None, None, None, None, None


def attention(q, k, v, index: Index, coords, rope_base=10000.0, scale=None, with_summaries=True,
              position_mode="axial"):
    """PACK3D attention with autograd support (position_mode: see make_attn)."""
    return Pack3DAttention.apply(q, k, v, index, coords, rope_base, scale, with_summaries, position_mode)


class Pack3DAttentionQKV(torch.autograd.Function):
    """Autograd wrapper over the fused-projection entry points: qkv [T, 3, H, D] -> out [T, H, D]."""

    @staticmethod
    def forward(ctx, qkv, index: Index, coords, rope_base=10000.0, scale=None, with_summaries=True,
                position_mode="axial"):
        qkv = qkv.contiguous()
        attn = make_attn(qkv.dtype, qkv.shape[2], qkv.shape[3], rope_base, scale, with_summaries, position_mode)
        need = workspace_bytes(index, attn, True)
        if need == 0:
            raise Pack3DError(E_UNSUPPORTED, load_library().pack3d_last_error().decode())
        ws = torch.empty(need, dtype=torch.uint8, device=qkv.device)
        out, lse = forward_qkv(index, qkv, coords, rope_base=rope_base, scale=scale, with_summaries=with_summaries,
                               workspace=ws, position_mode=position_mode)
        ctx.save_for_backward(qkv, out, lse, coords)
        ctx.index, ctx.workspace = index, ws
        ctx.opts = (rope_base, scale, with_summaries, position_mode)
        return out

    @staticmethod
    def backward(ctx, dout):
        qkv, out, lse, coords = ctx.saved_tensors
        rope_base, scale, with_summaries, position_mode = ctx.opts
        ws, ctx.workspace = ctx.workspace, None
        dqkv = backward_qkv(ctx.index, qkv, coords, out, lse, dout.contiguous(), rope_base=rope_base, scale=scale,
                            with_summaries=with_summaries, workspace=ws, reuse_forward=ws is not None,
                            position_mode=position_mode)
        return dqkv, None, None, None, None, None, None


def attention_qkv(qkv, index: Index, coords, rope_base=10000.0, scale=None, with_summaries=True,
                  position_mode="axial"):
    """PACK3D attention on a fused projection output qkv [T, 3, H, D], with autograd."""
    return Pack3DAttentionQKV.apply(qkv, index, coords, rope_base, scale, with_summaries, position_mode)
