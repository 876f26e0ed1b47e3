"""Host emulation of the memory accesses of bwd_dq's 32-column direct-copy kernel (k_bwd_dq32).

Two earlier direct-copy bwd_dq kernels raised illegal-address faults, only in position mode
"none", and the one place that mode changes addressing is the workspace layout: its
rotation table is one row, so every later array starts at another offset.  This test redoes,
in plain integer arithmetic, every address the new kernel forms for the geometry that
faulted (a 8x8x16 grid in 4x4x4 blocks, 2 volumes, 2 heads, D = 96, bf16) under the
workspace layout of each position mode, and checks that each one lies inside its buffer:
the 16-byte tile copies (source range against the buffer resource's extent and against the
workspace, LDS destination against the stage), the transposed LDS reads of the K tile, the
lse / delta reads and the dq row writes.  No GPU is involved.  (The kernel also runs only for
the axial and packed-1D modes; mode "none" keeps the register-staged kernel.)"""
import itertools

import pytest

B, H, D, DP = 2, 2, 96, 96
GRID, BLOCK = (8, 8, 16), (4, 4, 4)
BVOL, TILE, THREADS = 64, 64, 256
ES = 2  # bf16


def align(x, a=256):
    return (x + a - 1) // a * a


def workspace(mode):
    """Byte offsets of the workspace arrays (the layout of the library's workspace) for this
    geometry and position mode, and the backward total."""
    nb = [g // b for g, b in zip(GRID, BLOCK)]
    nblk = nb[0] * nb[1] * nb[2]
    nc, nblkp = nblk * BVOL, align(nblk, 64)
    trows, half = {"axial": (max(GRID), D // 6), "packed1d": (nc, D // 2), "none": (1, D // 2)}[mode]
    act, summ = B * H * nc * DP * ES, B * H * nblkp * DP * ES
    summ32 = B * H * nblkp * DP * 4
    chunks = max(1, min(nblk, 2048 // max(1, (nblkp // TILE) * H * B)))
    off, w = 0, {}
    for name, size in (("rope", 8 * trows * half), ("qrot", act), ("krot", act), ("vr", act), ("kbar", summ),
                       ("vbar", summ), ("doc", act), ("lsec", 4 * B * H * nc), ("delta", 4 * B * H * nc),
                       ("dkbar", summ32), ("dvbar", summ32), ("part_k", summ32 * chunks), ("part_v", summ32 * chunks)):
        w[name] = off
        off = align(off + size)
    w["total"] = off
    return w, nb, nblk, nc, nblkp


def swz(r):  # 16-byte chunk swizzle of a 96-column bf16 LDS row
    b2, b3 = (r >> 2) & 1, (r >> 3) & 1
    return b2 | ((b2 ^ b3) << 1)


def copy_chunks():
    """(LDS byte offset, tile row, logical 16-byte chunk) of every copy slot of a tile."""
    ch = DP // 8
    out = []
    for p in range(TILE * ch):   # slot p = round * 256 + thread
        r = p // ch
        c = (p % ch) ^ swz(r)
        out.append((16 * p, r, c))
    return out


def neighbours(nb, blk):
    bz, rem = divmod(blk, nb[1] * nb[2])
    by, bx = divmod(rem, nb[2])
    out = []
    for dz, dy, dx in itertools.product((-1, 0, 1), repeat=3):
        z, y, x = bz + dz, by + dy, bx + dx
        if 0 <= z < nb[0] and 0 <= y < nb[1] and 0 <= x < nb[2]:
            out.append((z * nb[1] + y) * nb[2] + x)
    return out


@pytest.mark.parametrize("mode", ["none", "axial", "packed1d"])
def test_every_access_of_the_direct_copy_dq_kernel_is_in_bounds(mode):
    w, nb, nblk, nc, nblkp = workspace(mode)
    tile_bytes = TILE * DP * ES
    slots = copy_chunks()
    assert all(0 <= lds + 16 <= tile_bytes for lds, _, _ in slots)
    for b, h in itertools.product(range(B), range(H)):
        bh = b * H + h
        for qb in range(nblk):
            local = neighbours(nb, qb)
            tiles = [("krot", "vr", blk * BVOL, nc) for blk in local]
            tiles += [("kbar", "vbar", ts * TILE, nblkp) for ts in range(nblkp // TILE)]
            for kname, vname, row0, rows in tiles:
                for name in (kname, vname):
                    base = w[name] + bh * rows * DP * ES        # the buffer resource's base
                    extent = rows * DP * ES                      # and its number of records
                    for _, r, c in slots:
                        off = ((row0 + r) * DP + 8 * c) * ES
                        assert 0 <= off and off + 16 <= extent, (mode, name, qb, r, c)
                        assert base + off + 16 <= w["total"]
            # lse2 and -delta of the workgroup's 64 queries
            for q in range(TILE):
                i = bh * nc + qb * BVOL + q
                assert 4 * i + 4 <= B * H * nc * 4
    # the transposed K reads: per lane two base offsets plus the asm block's byte offsets
    for kh, lane in itertools.product(range(2), range(64)):
        half, lane16, hi16 = lane >> 5, lane & 15, (lane >> 4) & 1

        def base(r15, c3):
            return r15 * DP + ((c3 ^ swz(r15)) << 3)

        def bases(r15):
            r, c = r15 + (lane16 >> 2), 4 * (lane16 & 3)
            return base(r, c >> 3) + (c & 7), base(r, 2 + (c >> 3)) + (c & 7)

        for r15 in (4 * half, 8 + 4 * half):
            even, odd = bases(r15)
            p = (odd if hi16 else even) + 32 * kh * DP
            for extra in (0, 64, 128, 3072, 3136, 3200):
                assert 0 <= 2 * p + extra and 2 * p + extra + 8 <= tile_bytes
    # the dq rows written by the epilogue: 96 values of one (token, head) row, 4-element pieces
    n_tok = GRID[0] * GRID[1] * GRID[2]
    for tok, hh in ((0, 0), (n_tok - 1, H - 1), (B * n_tok - 1, H - 1)):
        row = tok * H * D + hh * D
        for dt, jj, half in itertools.product(range(3), range(4), range(2)):
            assert row + 32 * dt + 8 * jj + 4 * half + 4 <= B * n_tok * H * D


def test_the_workspace_offsets_differ_by_mode_as_described():
    """Mode "none" moves every array 1,536 bytes down against axial at this geometry."""
    offs = {m: workspace(m)[0] for m in ("none", "axial", "packed1d")}
    assert offs["none"]["qrot"] == 512 and offs["axial"]["qrot"] == 2048
    assert offs["packed1d"]["qrot"] == align(8 * 1024 * 48)
