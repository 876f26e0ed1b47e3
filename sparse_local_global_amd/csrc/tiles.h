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

template <typename T> struct Pad;
template <> struct Pad<bf16> { static constexpr int row = 8, tr = 8, vec = 8; };
template <> struct Pad<float> { static constexpr int row = 4, tr = 4, vec = 4; };

// 64 rows x DP, head dim contiguous.
template <typename T, int DP> struct alignas(16) RowTile { T x[kTile][DP + Pad<T>::row]; };
// DP x 64, the 64 rows contiguous.
template <typename T, int DP> struct alignas(16) TrTile { T x[DP][kTile + Pad<T>::tr]; };

// The 16 register rows of a wave (B operand of score).
template <typename T, int DP> struct ColFrag;

template <int DP> struct ColFrag<bf16, DP> {
  bf16x8 b[DP / 32];
  // row: start of this lane's column row (DP elements), or ok = false for a zero row
  __device__ inline void load(const bf16* __restrict__ row, bool ok, int grp) {
#pragma unroll
    for (int s = 0; s < DP / 32; ++s) {
      if (ok) b[s] = *(const bf16x8*)(row + 32 * s + 8 * grp);
      else b[s] = bf16x8{};
    }
  }
};

template <int DP> struct ColFrag<float, DP> {
  float b[DP / 4];
  __device__ inline void load(const float* __restrict__ row, bool ok, int grp) {
#pragma unroll
    for (int s = 0; s < DP / 4; s += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (ok) x = *(const f32x4*)(row + grp * (DP / 4) + s);
      b[s] = x[0]; b[s + 1] = x[1]; b[s + 2] = x[2]; b[s + 3] = x[3];
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

// Cooperative 16-byte loads.  rowoff(r) = element offset of row r (r < valid), others zero.
template <typename T, int DP, typename RowOff>
__device__ inline void load_rows(RowTile<T, DP>& t, const T* __restrict__ src, int valid, RowOff rowoff) {
  constexpr int V = Pad<T>::vec;
  constexpr int chunks = kTile * DP / V;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    const int row = c / (DP / V), cc = (c - row * (DP / V)) * V;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (row < valid) x = *(const uint4*)(src + rowoff(row) + cc);
    *(uint4*)&t.x[row][cc] = x;
  }
}

// troff(d, r) = element offset of V consecutive rows r.. of column d (r a multiple of V, r < valid).
template <typename T, int DP, typename TrOff>
__device__ inline void load_tr(TrTile<T, DP>& t, const T* __restrict__ src, int valid, TrOff troff) {
  constexpr int V = Pad<T>::vec;
  constexpr int chunks = DP * kTile / V;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    const int d = c / (kTile / V), r = (c - d * (kTile / V)) * V;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (r < valid) x = *(const uint4*)(src + troff(d, r));
    *(uint4*)&t.x[d][r] = x;
  }
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
