// Matrix-core tile primitives shared by the attention kernels (forward and backward).
//
// Every contraction of the operator has one of two shapes, for a wave that owns
// 16 "columns" (queries in the query-major kernels, keys or summaries in the
// key-major ones) and streams 64 "rows" through LDS:
//   score:  s[r][c]   = sum_d  R[r][d] * C[c][d]        (R: 64 LDS rows, C: 16 register rows)
//   accum:  acc[d][c] += sum_r RT[d][r] * p[r][c]        (RT: the 64 rows transposed in LDS,
//                                                         p: a score tile in accumulator layout)
// The score tile leaves the matrix core with one column per lane (lane & 15) and
// rows 16*mt + 4*(lane >> 4) + i, which is exactly the B-operand layout the accum
// contraction needs, so scores never travel through LDS.
//   bf16: v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  In both operands k slot e of
//         lane group g is head dim 32s + 8g + e (score) or row 32c + 4g + e (e < 4) /
//         32c + 16 + 4g + (e - 4) (e >= 4) (accum).
//   fp32: v_mfma_f32_16x16x4_f32.  k index g is head dim g*DP/4 + s (score) or row
//         16mt + 4g + i (accum, one MFMA per i).
#pragma once

#include "layout.h"

namespace pack3d {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A global array addressed through a buffer resource (base in SGPRs, 32-bit byte
// offsets in VGPRs); reads at or past `bytes` return zero.
struct Src {
  __amdgpu_buffer_rsrc_t r;
  __device__ inline Src(const void* base, size_t bytes) {
    // num_records < 2^31, so the offset 0x80000000 used for padding rows is always out of range
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                          (int)(bytes > 0x7fffff00u ? 0x7fffff00u : bytes), 0x00020000);
  }
  __device__ inline uint4 load16(uint32_t byte_off) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Pad;
// Row pads keep the LDS reads of both contraction shapes free of bank conflicts on 32
// 4-byte banks: 208-byte K rows (16-byte reads, 8 lanes per cycle) and 136-byte V^T rows
// (8-byte reads, 16 lanes per cycle).
template <> struct Pad<bf16> { static constexpr int row = 8, tr = 4, vec = 8; };
template <> struct Pad<float> { static constexpr int row = 4, tr = 4, vec = 4; };

// 64 rows x DP, head dim contiguous.
template <typename T, int DP> struct alignas(16) RowTile { T x[kTile][DP + Pad<T>::row]; };
// DP x 64, the 64 rows contiguous.
template <typename T, int DP> struct alignas(16) TrTile { T x[DP][kTile + Pad<T>::tr]; };

// The 16 register rows of a wave (B operand of score).
template <typename T, int DP> struct ColFrag;

template <int DP> struct ColFrag<bf16, DP> {
  bf16x8 b[DP / 32];
  // row: start of this lane's column row (DP elements), or ok = false for a zero row;
  // every element is multiplied by `mul` (rounded back to bf16) when mul != 1
  __device__ inline void load(const bf16* __restrict__ row, bool ok, int grp, float mul = 1.0f) {
#pragma unroll
    for (int s = 0; s < DP / 32; ++s) {
      if (ok) b[s] = *(const bf16x8*)(row + 32 * s + 8 * grp);
      else b[s] = bf16x8{};
      if (mul != 1.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) b[s][e] = (bf16)((float)b[s][e] * mul);
      }
    }
  }
};

template <int DP> struct ColFrag<float, DP> {
  float b[DP / 4];
  __device__ inline void load(const float* __restrict__ row, bool ok, int grp, float mul = 1.0f) {
#pragma unroll
    for (int s = 0; s < DP / 4; s += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (ok) x = *(const f32x4*)(row + grp * (DP / 4) + s);
      b[s] = x[0] * mul; b[s + 1] = x[1] * mul; b[s + 2] = x[2] * mul; b[s + 3] = x[3] * mul;
    }
  }
};

template <int DP>
__device__ inline void score(const RowTile<bf16, DP>& t, const ColFrag<bf16, DP>& f, f32x4 (&s)[4], int col, int grp) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < DP / 32; ++k) {
      const bf16x8 a = *(const bf16x8*)&t.x[16 * mt + col][32 * k + 8 * grp];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, f.b[k], acc, 0, 0, 0);
    }
    s[mt] = acc;
  }
}

template <int DP>
__device__ inline void score(const RowTile<float, DP>& t, const ColFrag<float, DP>& f, f32x4 (&s)[4], int col, int grp) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < DP / 4; k += 4) {
      const f32x4 a = *(const f32x4*)&t.x[16 * mt + col][grp * (DP / 4) + k];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], f.b[k + e], acc, 0, 0, 0);
    }
    s[mt] = acc;
  }
}

template <int DP>
__device__ inline void accum(const TrTile<bf16, DP>& t, const f32x4 (&p)[4], f32x4 (&acc)[DP / 16], int col, int grp) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = (bf16)p[2 * c][e];
      b[e + 4] = (bf16)p[2 * c + 1][e];
    }
#pragma unroll
    for (int dt = 0; dt < DP / 16; ++dt) {
      const bf16x4 lo = *(const bf16x4*)&t.x[16 * dt + col][32 * c + 4 * grp];
      const bf16x4 hi = *(const bf16x4*)&t.x[16 * dt + col][32 * c + 16 + 4 * grp];
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[dt], 0, 0, 0);
    }
  }
}

template <int DP>
__device__ inline void accum(const TrTile<float, DP>& t, const f32x4 (&p)[4], f32x4 (&acc)[DP / 16], int col, int grp) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int dt = 0; dt < DP / 16; ++dt) {
      const f32x4 a = *(const f32x4*)&t.x[16 * dt + col][16 * mt + 4 * grp];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], p[mt][i], acc[dt], 0, 0, 0);
    }
  }
}

// Register-staged tile copies, for a software pipeline: fetch() issues every 16-byte
// global load of a tile at once (no dependency between them), store() writes them to
// LDS later, so the loads of tile t+1 are in flight while tile t is computed.
// rowoff(r) = element offset of row r (r < valid); other rows are zero.
template <typename T, int DP>
struct RowRegs {
  static constexpr int V = Pad<T>::vec;
  static constexpr int n = kTile * DP / V / kThreads;
  static_assert(kTile * DP / V % kThreads == 0, "tile chunks must spread evenly");
  uint4 r[n];
  template <typename RowOff>
  __device__ inline void fetch(const Src& src, int valid, RowOff rowoff) {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = c / (DP / V), cc = (c - row * (DP / V)) * V;
      // rows past `valid` read past the end of the buffer, which returns zero
      const uint32_t off = row < valid ? (uint32_t)(rowoff(row) + cc) * (uint32_t)sizeof(T) : 0x80000000u;
      r[i] = src.load16(off);
    }
  }
  // Tile whose rows are contiguous from element `base` (uniform across the workgroup).
  __device__ inline void fetch_at(const Src& src, uint32_t base) {
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base * (uint32_t)sizeof(T)));
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      r[i] = src.load16(b + (uint32_t)c * (uint32_t)(V * sizeof(T)));  // row-major: chunk c at c * V
    }
  }
  __device__ inline void store(RowTile<T, DP>& t) const {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int row = c / (DP / V), cc = (c - row * (DP / V)) * V;
      *(uint4*)&t.x[row][cc] = r[i];
    }
  }
};

// troff(d, r) = element offset of V consecutive rows r.. of column d (r a multiple of V,
// r < valid); other rows are zero.
template <typename T, int DP>
struct TrRegs {
  static constexpr int V = Pad<T>::vec;
  static constexpr int n = DP * kTile / V / kThreads;
  static_assert(DP * kTile / V % kThreads == 0, "tile chunks must spread evenly");
  uint4 r[n];
  template <typename TrOff>
  __device__ inline void fetch(const Src& src, int valid, TrOff troff) {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int d = c / (kTile / V), rr = (c - d * (kTile / V)) * V;
      const uint32_t off = rr < valid ? (uint32_t)troff(d, rr) * (uint32_t)sizeof(T) : 0x80000000u;
      r[i] = src.load16(off);
    }
  }
  // Tile whose column d starts at element base + d * stride (base uniform).
  __device__ inline void fetch_at(const Src& src, uint32_t base, uint32_t stride) {
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base * (uint32_t)sizeof(T)));
    const uint32_t sb = stride * (uint32_t)sizeof(T);
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int d = c / (kTile / V), rr = (c - d * (kTile / V)) * V;
      r[i] = src.load16(b + (uint32_t)d * sb + (uint32_t)(rr * sizeof(T)));
    }
  }
  __device__ inline void store(TrTile<T, DP>& t) const {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int d = c / (kTile / V), rr = (c - d * (kTile / V)) * V;
      // rows are 8-byte aligned (not 16): two 8-byte stores
      uint2* p = (uint2*)&t.x[d][rr];
      p[0] = make_uint2(r[i].x, r[i].y);
      p[1] = make_uint2(r[i].z, r[i].w);
    }
  }
};

// Rows j0 .. j0+63 of the virtual concatenation of the blocks in `list` (bvol rows each,
// canonical order).  When bvol is a multiple of 64 the tile lies inside one block and
// every row offset follows from one base; otherwise each row finds its block.
struct VirtualRows {
  const int* list;
  int bvol, j0;
  bool one_block;
  int blk0, off0;  // block and offset of tile row 0 when one_block
  __device__ inline VirtualRows(const int* l, int bv, int j) : list(l), bvol(bv), j0(j) {
    one_block = (bv & 63) == 0;
    if (one_block) {
      const int q = j / bv;
      blk0 = l[q];
      off0 = j - q * bv;
    } else {
      blk0 = off0 = 0;
    }
  }
  // canonical row of tile row r
  __device__ inline int row(int r) const {
    if (one_block) return blk0 * bvol + off0 + r;
    const int j = j0 + r, q = j / bvol;
    return list[q] * bvol + (j - q * bvol);
  }
  // offset of (column d, tile row r) in a block-transposed array [nblk][dp][bvol]
  __device__ inline int tr(int d, int r, int dp) const {
    if (one_block) return (blk0 * dp + d) * bvol + off0 + r;
    const int j = j0 + r, q = j / bvol;
    return (list[q] * dp + d) * bvol + (j - q * bvol);
  }
};

// Workgroups are dealt to the 8 XCDs round-robin by linear id.  Map linear id L to a
// logical tile so that each XCD walks a contiguous range of logical tiles: neighbouring
// tiles share their key / value tiles, which then stay in that XCD's L2.
__device__ inline int xcd_remap(int L, int total) {
  if (total % 8) return L;
  return (L & 7) * (total >> 3) + (L >> 3);
}

// Compact the neighbour-table row of block `blk` (wave 0 only); returns the count in *n.
__device__ inline void compact_neighbours(const int32_t* __restrict__ nbr_row, int slots, int* list, int* n) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c = 0; c < slots; c += 64) {
    const int s = c + lane;
    const int id = s < slots ? nbr_row[s] : -1;
    const uint64_t m = __ballot(id >= 0);
    const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
    if (id >= 0) list[pos] = id;
    base += __popcll(m);
  }
  if (lane == 0) *n = base;
}

}  // namespace pack3d
