"""The C-ABI library builds, loads and exports every entry point declared in include/pack3d.h.

Host-side checks only: no call here reaches a GPU (argument errors are rejected
before any HIP call).
"""
import ctypes
import os
import re

import pytest
import torch

import sparse_local_global_amd.pack3d as p3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pack3d.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pack3d_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = p3.load_library()
    names = _declared_functions()
    assert len(names) == 18
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) <= set(p3.EXPORTS)


def test_exported_symbols_in_dynamic_table():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", p3.LIB_PATH], capture_output=True, text=True).stdout
    for name in _declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_last_error():
    lib = p3.load_library()
    assert lib.pack3d_version() == 104
    assert isinstance(lib.pack3d_last_error(), bytes)


def test_index_bytes_depends_only_on_layout():
    assert p3.index_bytes(2, 65536, (4, 4, 4), 1) > 0
    nblk, slots = 1024, 27
    expect = 0
    # geom, offsets, token_block, canon, perm, nbr, block counts, occupancy bits, empty-block bits
    for count in (2 * 10, 3, 2 * 65536, 2 * 65536, 2 * 65536, 2 * nblk * slots, 2 * nblk, 2 * 65536 // 32,
                  2 * nblk // 32):
        expect = (expect + 4 * count + 255) // 256 * 256
    assert p3.index_bytes(2, 65536, (4, 4, 4), 1) == expect
    assert p3.index_bytes(1, 100, (4, 4, 4), 1) == 0      # 100 tokens cannot tile into 64-token blocks
    assert p3.index_bytes(1, 512, (2, 2, 2), -1) == 0
    assert p3.index_bytes(1, 512, (0, 2, 2), 1) == 0
    assert p3.index_bytes(0, 512, (2, 2, 2), 1) == 0


def test_build_index_argument_errors_return_codes():
    lib = p3.load_library()
    pk = p3.Packing(1, 512, 0)
    bs = (ctypes.c_int32 * 3)(2, 2, 2)
    h = ctypes.c_void_p()
    st = lib.pack3d_build_index(None, ctypes.byref(pk), bs, 1, ctypes.c_void_p(256), 1 << 20, None, ctypes.byref(h))
    assert st == p3.E_INVALID and b"null" in lib.pack3d_last_error()
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk), bs, -1, ctypes.c_void_p(256), 1 << 20,
                                None, ctypes.byref(h))
    assert st == p3.E_INVALID
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk), bs, 9, ctypes.c_void_p(256), 1 << 20,
                                None, ctypes.byref(h))
    assert st == p3.E_UNSUPPORTED
    pk2 = p3.Packing(1, 500, 0)
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk2), bs, 1, ctypes.c_void_p(256), 1 << 20,
                                None, ctypes.byref(h))
    assert st == p3.E_COORDS
    bs3 = (ctypes.c_int32 * 3)(1, 1, 3)                      # 3-token blocks: not a multiple of 8
    pk3 = p3.Packing(1, 48, 0)
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk3), bs3, 1, ctypes.c_void_p(256), 1 << 20,
                                None, ctypes.byref(h))
    assert st == p3.E_UNSUPPORTED
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk), bs, 1, ctypes.c_void_p(256), 16,
                                None, ctypes.byref(h))
    assert st == p3.E_WORKSPACE
    assert not h.value


def test_forward_argument_errors_return_codes():
    lib = p3.load_library()
    at = p3.Attn(p3.BF16, 8, 96, 10000.0, 0.0, 1)
    st = lib.pack3d_forward(None, ctypes.byref(at), *([None] * 6), None, 0, None)
    assert st == p3.E_INVALID
    assert lib.pack3d_workspace_bytes(None, ctypes.byref(at), 0) == 0
    st = lib.pack3d_backward(None, ctypes.byref(at), *([None] * 10), None, 0, 0, None)
    assert st == p3.E_INVALID


def test_position_mode_argument():
    at = p3.make_attn(torch.bfloat16, 8, 96, position_mode="packed1d")
    assert at.position_mode == 1
    assert p3.make_attn(torch.float32, 2, 12).position_mode == 0
    with pytest.raises(p3.Pack3DError) as e:
        p3.make_attn(torch.float32, 2, 12, position_mode="sequence")
    assert e.value.status == p3.E_INVALID


def test_ragged_and_varlen_index_bytes():
    full = p3.index_bytes(2, 65536, (4, 4, 4), 1)
    # varlen offsets describing the same two volumes size the same tables
    assert p3.index_bytes(2, 0, (4, 4, 4), 1, offsets=[0, 65536, 131072]) == full
    # ragged: sized by max_blocks, not by the token counts
    assert p3.index_bytes(2, 65536, (4, 4, 4), 1, ragged=True, max_blocks=1024) == full
    assert p3.index_bytes(2, 65536, (4, 4, 4), 1, ragged=True, max_blocks=2048) > full
    assert p3.index_bytes(1, 100, (4, 4, 4), 1, ragged=True, max_blocks=4) > 0   # any token count
    assert p3.index_bytes(1, 100, (4, 4, 4), 1, ragged=True) == 0                # needs max_blocks
    assert p3.index_bytes(2, 0, (2, 2, 2), 1, offsets=[0, 64, 40]) == 0          # decreasing offsets
    assert p3.index_bytes(2, 0, (2, 2, 2), 1, offsets=[0, 64, 64]) == 0          # empty volume
    assert p3.index_bytes(2, 0, (2, 2, 2), 1, offsets=[8, 64, 72]) == 0          # must start at 0
    assert p3.index_bytes(2, 0, (4, 4, 4), 1, offsets=[0, 64, 100]) == 0         # 36 tokens without ragged


def test_measure_blocks_argument_errors():
    lib = p3.load_library()
    pk = p3._packing(1, 512, ragged=True)
    bs = (ctypes.c_int32 * 3)(2, 2, 2)
    out = ctypes.c_int32()
    st = lib.pack3d_measure_blocks(None, ctypes.byref(pk), bs, ctypes.c_void_p(256), 64, None, ctypes.byref(out))
    assert st == p3.E_INVALID
    st = lib.pack3d_measure_blocks(ctypes.c_void_p(256), ctypes.byref(pk), bs, ctypes.c_void_p(256), 8, None,
                                   ctypes.byref(out))
    assert st == p3.E_WORKSPACE and b"scratch" in lib.pack3d_last_error()
    bs3 = (ctypes.c_int32 * 3)(1, 1, 3)
    st = lib.pack3d_measure_blocks(ctypes.c_void_p(256), ctypes.byref(pk), bs3, ctypes.c_void_p(256), 64, None,
                                   ctypes.byref(out))
    assert st == p3.E_UNSUPPORTED


def test_ragged_build_needs_max_blocks():
    lib = p3.load_library()
    pk = p3._packing(1, 100, ragged=True)
    bs = (ctypes.c_int32 * 3)(2, 2, 2)
    h = ctypes.c_void_p()
    st = lib.pack3d_build_index(ctypes.c_void_p(256), ctypes.byref(pk), bs, 1, ctypes.c_void_p(256), 1 << 20,
                                None, ctypes.byref(h))
    assert st == p3.E_INVALID and b"max_blocks" in lib.pack3d_last_error()


def test_fused_entry_points_argument_errors():
    lib = p3.load_library()
    at = p3.Attn(p3.BF16, 8, 96, 10000.0, 0.0, 1)
    st = lib.pack3d_forward_qkv(None, ctypes.byref(at), None, None, None, None, None, 0, None)
    assert st == p3.E_INVALID and b"null" in lib.pack3d_last_error()
    st = lib.pack3d_backward_qkv(None, ctypes.byref(at), None, None, None, None, None, None, None, 0, 0, None)
    assert st == p3.E_INVALID
    odd = p3.Attn(p3.BF16, 1, 6, 10000.0, 0.0, 1)            # one head of 6 bf16: 12 bytes per head block
    st = lib.pack3d_forward_qkv(None, ctypes.byref(odd), ctypes.c_void_p(256), None, None, None, None, 0, None)
    assert st == p3.E_UNSUPPORTED and b"16 bytes" in lib.pack3d_last_error()
    st = lib.pack3d_forward_qkv(None, None, ctypes.c_void_p(256), None, None, None, None, 0, None)
    assert st == p3.E_INVALID


ABI_C = os.path.join(ROOT, "tests", "abi", "abi_consumer.c")


def _gcc(out, *extra):
    import subprocess
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), ABI_C, "-o", out, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _run(exe, *args):
    import subprocess
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    return dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())


def test_c_layout_matches_the_binding(tmp_path):
    """The header compiled by a C compiler lays out every struct and enum exactly as the
    ctypes declarations of the binding assume."""
    exe = str(tmp_path / "abi_layout")
    _gcc(exe)
    got = _run(exe)
    structs = {"pack3d_packing": p3.Packing, "pack3d_attn": p3.Attn, "pack3d_tables": p3.Tables,
               "pack3d_views": p3.Views}
    for cname, cls in structs.items():
        assert int(got[f"sizeof.{cname}"]) == ctypes.sizeof(cls), cname
        fields = [f[0] for f in cls._fields_]
        c_fields = sorted(k.split(".")[2] for k in got if k.startswith(f"offsetof.{cname}."))
        assert sorted(fields) == c_fields, cname
        for f in fields:
            assert int(got[f"offsetof.{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)
    enums = {"PACK3D_OK": p3.OK, "PACK3D_E_INVALID": p3.E_INVALID, "PACK3D_E_COORDS": p3.E_COORDS,
             "PACK3D_E_UNSUPPORTED": p3.E_UNSUPPORTED, "PACK3D_E_WORKSPACE": p3.E_WORKSPACE,
             "PACK3D_E_HIP": p3.E_HIP, "PACK3D_F32": p3.F32, "PACK3D_BF16": p3.BF16,
             "PACK3D_ORDER_ANY": p3.ORDERS["any"], "PACK3D_ORDER_RASTER": p3.ORDERS["raster"],
             "PACK3D_ORDER_MORTON": p3.ORDERS["morton"], "PACK3D_ORDER_BLOCK_CONTIGUOUS": p3.ORDERS["block"],
             "PACK3D_ORDER_RANDOM": p3.ORDERS["random"], "PACK3D_POS_AXIAL": p3.POSITION_MODES["axial"],
             "PACK3D_POS_PACKED_1D": p3.POSITION_MODES["packed1d"], "PACK3D_POS_NONE": p3.POSITION_MODES["none"]}
    c_enums = {k.split(".", 1)[1] for k in got if k.startswith("enum.")}
    assert c_enums == set(enums)
    for name, value in enums.items():
        assert int(got[f"enum.{name}"]) == value, name


def test_c_program_links_and_calls_the_library(tmp_path):
    """A C program linked against libpack3d.so calls the entry points that need no GPU and
    gets the same answers as the binding."""
    p3.load_library()
    libdir = os.path.dirname(p3.LIB_PATH)
    exe = str(tmp_path / "abi_call")
    _gcc(exe, "-DPACK3D_LINKED", "-L", libdir, "-lpack3d", f"-Wl,-rpath,{libdir}")
    got = _run(exe, "call")
    assert int(got["call.version"]) == p3.load_library().pack3d_version()
    assert int(got["call.index_bytes"]) == p3.index_bytes(2, 65536, (4, 4, 4), 1) > 0
    assert int(got["call.index_bytes_bad"]) == 0
    assert int(got["call.build_index_null"]) == p3.E_INVALID
    assert got["call.build_index_null_message"] == "set"
    assert got["call.handle_null"] == "1"
