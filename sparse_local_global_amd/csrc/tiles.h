// Matrix-core tile primitives shared by the attention kernels (forward and backward).
//
// Every contraction of the operator has one of two shapes, for a wave that owns
// 16 "columns" (queries in the query-major kernels, keys or summaries in the
// key-major ones) and streams 64 "rows" through LDS:
//   score:  s[r][c]   = sum_d  X[r][d] * C[c][d]        (X: 64 LDS rows, C: 16 register rows)
//   accum:  acc[d][c] += sum_r X[r][d] * p[r][c]         (X: 64 LDS rows, p: a score tile
//                                                         in accumulator layout)
// Both read the same row-major tile X[64][DP].  The score tile leaves the matrix core
// with one column per lane (lane & 15) and rows 16*mt + 4*(lane >> 4) + i, which is the
// B-operand layout the accum contraction needs, so scores never travel through LDS.
//   bf16: v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  score: k slot e of lane group g
//         is head dim 32s + 8g + e.  accum: k slot e is row 32c + 4g + e (e < 4) or
//         32c + 16 + 4g + (e - 4) (e >= 4); its A operand (rows of column d) is read with
//         the LDS transpose load ds_read_b64_tr_b16, which hands lane i of a 16-lane group
//         the 4 rows r0..r0+3 of column c0 + i when lane j points at row r0 + j/4,
//         columns c0 + 4*(j%4) .. +3.
//   fp32: v_mfma_f32_16x16x4_f32.  score: k index g is head dim g*DP/4 + s; accum: k
//         index g is row 16mt + 4g + i (one MFMA per i, A read as single dwords).
#pragma once

#include <type_traits>

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

// LDS row tile X[64][DP] (head dim contiguous).
//   bf16: rows of RS elements; the 16-byte chunk c of row r is stored at chunk
//   c ^ swz(r).  gfx950's LDS has 64 four-byte banks.  A 64-bit read (plain or
//   transposing) serves 32 consecutive lanes per pass.  A 128-bit read serves 16 lanes
//   per pass, namely four 4-lane quads: those with equal lane bit 5 and equal parity of
//   lane bits 2..4 (quads {0,3,5,6}, {1,2,4,7} and the same +8); both facts were
//   measured with the LDS bank-conflict counter on two-lane and whole-wave patterns.
//   Under that model the score reads (16- and 32-column waves), both transpose reads and
//   the row stores are all conflict-free for
//     DP = 32, 96:  RS = DP,      swz(r) = bit2(r) + 2*(bit2(r) ^ bit3(r))
//   and for DP = 64, 128 (RS = DP + 16, swz(r) = 2*bit3(r) + bit0(r)) the 16-column
//   score reads conflict 2-way.
//   fp32: rows of DP + 4 floats, no swizzle.
template <typename T, int DP> struct TileGeom;
template <int DP> struct TileGeom<bf16, DP> {
  static constexpr bool odd = (DP / 32) & 1;
  static constexpr int RS = odd ? DP : DP + 16;
  static constexpr int vec = 8;
  __device__ static inline int swz(int r) {
    return odd ? (((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1)) : ((((r >> 3) & 1) << 1) | (r & 1));
  }
  // element offset of chunk c (8 elements) of row r
  __device__ static inline int chunk(int r, int c) { return r * RS + ((c ^ swz(r)) << 3); }
  // swz depends on r & 15 only and is below 4, so it permutes chunks within aligned
  // groups of four: chunk(r, c) = base(r & 15, c & 3) + off(r & ~15, c & ~3).  The
  // readers below keep base() in a register per lane and pass off() as an immediate.
  __device__ static inline int base(int r15, int c3) { return r15 * RS + ((c3 ^ swz(r15)) << 3); }
  __device__ static constexpr int off(int rhi, int chi) { return rhi * RS + (chi << 3); }
};
template <int DP> struct TileGeom<float, DP> {
  static constexpr int RS = DP + 4;
  static constexpr int vec = 4;
  __device__ static inline int chunk(int r, int c) { return r * RS + (c << 2); }
};

template <typename T, int DP> struct alignas(16) RowTile { T x[kTile * TileGeom<T, DP>::RS]; };

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

// score_acc adds the scores onto the values s holds (an offset per element); score
// starts from zero.
template <int DP>
__device__ inline void score_acc(const RowTile<bf16, DP>& t, const ColFrag<bf16, DP>& f, f32x4 (&s)[4], int col,
                                 int grp) {
  using G = TileGeom<bf16, DP>;
  const bf16* b0 = t.x + G::base(col, grp);  // row 16mt + col, chunk 4k + grp
  // k outer, row tile inner: the four accumulation chains interleave
#pragma unroll
  for (int k = 0; k < DP / 32; ++k) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const bf16x8 a = *(const bf16x8*)(b0 + G::off(16 * mt, 4 * k));
      s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, f.b[k], s[mt], 0, 0, 0);
    }
  }
}

template <int DP>
__device__ inline void score_acc(const RowTile<float, DP>& t, const ColFrag<float, DP>& f, f32x4 (&s)[4], int col,
                                 int grp) {
  using G = TileGeom<float, DP>;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 acc = s[mt];
#pragma unroll
    for (int k = 0; k < DP / 4; k += 4) {
      const f32x4 a = *(const f32x4*)&t.x[(16 * mt + col) * G::RS + grp * (DP / 4) + k];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], f.b[k + e], acc, 0, 0, 0);
    }
    s[mt] = acc;
  }
}

template <typename T, int DP>
__device__ inline void score(const RowTile<T, DP>& t, const ColFrag<T, DP>& f, f32x4 (&s)[4], int col, int grp) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  score_acc(t, f, s, col, grp);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16 lds_bf16;

// Transpose read: lane j of a 16-lane group points at row r0 + j/4, columns
// c0 + 4(j%4) .. +3 (c0 a multiple of 16), and receives rows r0 .. r0+3 of column c0 + j.
// column_bases() gives the lane's element offsets for r0 & 15 = r15 and c0 an even /
// odd multiple of 16; G::off(r0 & ~15, 4 * (c0 / 32)) completes the address.
struct ColumnBases {
  int even;  // element offset in the tile for c0 = 32n
  int odd;   // for c0 = 32n + 16
};
template <int DP>
__device__ inline ColumnBases column_bases(int r15, int lane16) {
  using G = TileGeom<bf16, DP>;
  const int r = r15 + (lane16 >> 2);  // r15: a multiple of 4 below 16
  const int c = 4 * (lane16 & 3);     // column of this lane's piece within c0 .. c0+15
  return {G::base(r, c >> 3) + (c & 7), G::base(r, 2 + (c >> 3)) + (c & 7)};
}
// Element offsets (not pointers) select the lane's base, so every LDS address stays a
// plain offset from the tile object.
template <int DP>
__device__ inline bf16x4 read_tr(const RowTile<bf16, DP>& t, int off) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_bf16*)(t.x + off));
  return __builtin_bit_cast(bf16x4, v);
}

template <int DP>
__device__ inline void accum(const RowTile<bf16, DP>& t, const f32x4 (&p)[4], f32x4 (&acc)[DP / 16], int col, int grp) {
  using G = TileGeom<bf16, DP>;
  const ColumnBases cb = column_bases<DP>(4 * grp, col);  // rows 32c (+16) + 4grp + col/4
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
      const int cp = dt & 1 ? cb.odd : cb.even;  // columns 16dt ..
      const bf16x4 lo = read_tr(t, cp + G::off(32 * c, 4 * (dt >> 1)));
      const bf16x4 hi = read_tr(t, cp + G::off(32 * c + 16, 4 * (dt >> 1)));
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[dt], 0, 0, 0);
    }
  }
}

template <int DP>
__device__ inline void accum(const RowTile<float, DP>& t, const f32x4 (&p)[4], f32x4 (&acc)[DP / 16], int col, int grp) {
  using G = TileGeom<float, DP>;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * grp + i;
#pragma unroll
      for (int dt = 0; dt < DP / 16; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.x[r * G::RS + 16 * dt + col], p[mt][i], acc[dt], 0, 0, 0);
    }
  }
}

// ---- 32-column waves (bf16): v_mfma_f32_32x32x16_bf16 ------------------------------
// A wave owns 32 columns (lane & 31) and the two lane halves h = lane >> 5 split every
// 16-wide contraction step: k slot e of half h is head dim 16s + 8h + e (score) or row
// 16s + 4h + e (e < 4) / 16s + 8 + 4h + (e - 4) (e >= 4) (accum).  A 32x32 accumulator
// holds element (row 8*(i/4) + 4h + i%4, column lane & 31) in slot i.
typedef __attribute__((ext_vector_type(16))) float f32x16;

template <int DP> struct ColFrag32 {
  bf16x8 b[DP / 16];
  __device__ inline void load(const bf16* __restrict__ row, bool ok, int half) {
#pragma unroll
    for (int s = 0; s < DP / 16; ++s) {
      if (ok) b[s] = *(const bf16x8*)(row + 16 * s + 8 * half);
      else b[s] = bf16x8{};
    }
  }
};

// s[mt][i] = score of tile row 32mt + 8(i/4) + 4h + i%4 against column (lane & 31)
template <int DP>
__device__ inline void score32(const RowTile<bf16, DP>& t, const ColFrag32<DP>& f, f32x16 (&s)[2], int col, int half) {
  using G = TileGeom<bf16, DP>;
  // row 32mt + col, chunk 2k + half: one base per parity of k
  const bf16* be = t.x + G::base(col & 15, half) + G::off(col & 16, 0);
  const bf16* bo = t.x + G::base(col & 15, 2 + half) + G::off(col & 16, 0);
  // k outer, row tile inner: the two accumulation chains interleave
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int k = 0; k < DP / 16; ++k) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 a = *(const bf16x8*)((k & 1 ? bo : be) + G::off(32 * mt, 4 * (k >> 1)));
      s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, f.b[k], s[mt], 0, 0, 0);
    }
  }
}

// acc[dt][i] += sum_r X[r][32dt + 8(i/4) + 4h + i%4] * p[r][lane & 31]
template <int DP>
__device__ inline void accum32(const RowTile<bf16, DP>& t, const f32x16 (&p)[2], f32x16 (&acc)[DP / 32], int lane,
                               int half) {
  using G = TileGeom<bf16, DP>;
  const int lane16 = lane & 15, hi16 = (lane >> 4) & 1;
  // rows 16s + 4h (+8) + lane16/4, columns 32dt + 16hi16 + lane16
  const ColumnBases c0 = column_bases<DP>(4 * half, lane16), c8 = column_bases<DP>(8 + 4 * half, lane16);
  const int p0 = hi16 ? c0.odd : c0.even;
  const int p8 = hi16 ? c8.odd : c8.even;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // rows 16s + 4h + e (e < 4) and 16s + 8 + 4h + (e - 4): accumulator slots 8(s%2) + e
    const f32x16& ps = p[s >> 1];
    const int i0 = 8 * (s & 1);
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)ps[i0 + e];
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      const bf16x4 lo = read_tr(t, p0 + G::off(16 * s, 4 * dt));
      const bf16x4 hi = read_tr(t, p8 + G::off(16 * s, 4 * dt));
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[dt], 0, 0, 0);
    }
  }
}

// One 32-row block (rows 32mt .. 32mt+31) of two independent score tiles at once
// (the two accumulation chains interleave): s1 from t1 and f1, s2 from t2 and f2,
// slot i = row 32mt + 8(i/4) + 4h + i%4 against column (lane & 31).
// s2 starts from init2 (an offset per element), s1 from zero.
template <int DP>
__device__ inline void score32_pair(const RowTile<bf16, DP>& t1, const ColFrag32<DP>& f1, f32x16& s1,
                                    const RowTile<bf16, DP>& t2, const ColFrag32<DP>& f2, f32x16& s2, int col,
                                    int half, int mt, const f32x16& init2 = f32x16{}) {
  using G = TileGeom<bf16, DP>;
  const int be = G::base(col & 15, half) + G::off(col & 16, 0);
  const int bo = G::base(col & 15, 2 + half) + G::off(col & 16, 0);
  s1 = f32x16{};
  s2 = init2;
#pragma unroll
  for (int k = 0; k < DP / 16; ++k) {
    const int o = (k & 1 ? bo : be) + G::off(32 * mt, 4 * (k >> 1));
    const bf16x8 a1 = *(const bf16x8*)(t1.x + o);
    const bf16x8 a2 = *(const bf16x8*)(t2.x + o);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, f1.b[k], s1, 0, 0, 0);
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, f2.b[k], s2, 0, 0, 0);
  }
}

// score32_pair with its LDS reads scheduled NPRE ahead of the products that use them: the
// first NPRE reads are issued together, then each product is followed by the next read.
template <int DP, int NPRE>
__device__ inline void score32_pair_ahead(const RowTile<bf16, DP>& t1, const ColFrag32<DP>& f1, f32x16& s1,
                                          const RowTile<bf16, DP>& t2, const ColFrag32<DP>& f2, f32x16& s2, int col,
                                          int half, int mt) {
  using G = TileGeom<bf16, DP>;
  constexpr int NK = DP / 16, NR = 2 * NK;
  constexpr int NA = NPRE < NR ? NPRE : NR;  // reads ahead
  static_assert(NA > 0, "reads ahead");
  const int be = G::base(col & 15, half) + G::off(col & 16, 0);
  const int bo = G::base(col & 15, 2 + half) + G::off(col & 16, 0);
  bf16x8 a1[NK], a2[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int o = (k & 1 ? bo : be) + G::off(32 * mt, 4 * (k >> 1));
    a1[k] = *(const bf16x8*)(t1.x + o);
    a2[k] = *(const bf16x8*)(t2.x + o);
  }
  s1 = f32x16{};
  s2 = f32x16{};
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[k], f1.b[k], s1, 0, 0, 0);
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[k], f2.b[k], s2, 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NR - NA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NA, 0);
}

// score32_rows with its LDS reads scheduled NPRE ahead of the products that use them.
template <int DP, int NPRE>
__device__ inline void score32_rows_ahead(const RowTile<bf16, DP>& t, const ColFrag32<DP>& f, f32x16& s, int col,
                                          int half, int mt) {
  using G = TileGeom<bf16, DP>;
  constexpr int NK = DP / 16;
  constexpr int NA = NPRE < NK ? NPRE : NK;
  const int be = G::base(col & 15, half) + G::off(col & 16, 0);
  const int bo = G::base(col & 15, 2 + half) + G::off(col & 16, 0);
  bf16x8 a[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) a[k] = *(const bf16x8*)(t.x + (k & 1 ? bo : be) + G::off(32 * mt, 4 * (k >> 1)));
  s = f32x16{};
#pragma unroll
  for (int k = 0; k < NK; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], f.b[k], s, 0, 0, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, NA, 0);
#pragma unroll
  for (int i = 0; i < NK - NA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NA, 0);
}

// Rows 32mt .. 32mt+31 of one score tile: slot i = row 32mt + 8(i/4) + 4h + i%4 against
// column (lane & 31).
template <int DP>
__device__ inline void score32_rows(const RowTile<bf16, DP>& t, const ColFrag32<DP>& f, f32x16& s, int col, int half,
                                    int mt) {
  using G = TileGeom<bf16, DP>;
  const int be = G::base(col & 15, half) + G::off(col & 16, 0);
  const int bo = G::base(col & 15, 2 + half) + G::off(col & 16, 0);
  s = f32x16{};
#pragma unroll
  for (int k = 0; k < DP / 16; ++k) {
    const bf16x8 a = *(const bf16x8*)(t.x + (k & 1 ? bo : be) + G::off(32 * mt, 4 * (k >> 1)));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, f.b[k], s, 0, 0, 0);
  }
}

// acc[dt][i] += sum over rows r of block mt of X[r][32dt + 8(i/4) + 4h + i%4] * p[r][lane & 31],
// p in the slot layout of score32_pair.
template <int DP>
__device__ inline void accum32_rows(const RowTile<bf16, DP>& t, const f32x16& p, f32x16 (&acc)[DP / 32], int lane,
                                    int half, int mt) {
  using G = TileGeom<bf16, DP>;
  const int lane16 = lane & 15, hi16 = (lane >> 4) & 1;
  const ColumnBases c0 = column_bases<DP>(4 * half, lane16), c8 = column_bases<DP>(8 + 4 * half, lane16);
  const int p0 = hi16 ? c0.odd : c0.even;
  const int p8 = hi16 ? c8.odd : c8.even;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // rows 32mt + 16s + 4h + e (e < 4) and 32mt + 16s + 8 + 4h + (e - 4): slots 8s + e
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)p[8 * s + e];
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      const bf16x4 lo = read_tr(t, p0 + G::off(32 * mt + 16 * s, 4 * dt));
      const bf16x4 hi = read_tr(t, p8 + G::off(32 * mt + 16 * s, 4 * dt));
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[dt], 0, 0, 0);
    }
  }
}

// The A operands of accum32_rows (rows 32mt .. 32mt+31 of tile t, read with the LDS
// transpose load) held in registers, so the reads can happen at a chosen point.
template <int DP>
struct RowsFrag32 {
  bf16x8 a[2][DP / 32];
};

template <int DP>
__device__ inline void read_rows32(const RowTile<bf16, DP>& t, RowsFrag32<DP>& v, int lane, int half, int mt) {
  using G = TileGeom<bf16, DP>;
  const int lane16 = lane & 15, hi16 = (lane >> 4) & 1;
  const ColumnBases c0 = column_bases<DP>(4 * half, lane16), c8 = column_bases<DP>(8 + 4 * half, lane16);
  const int p0 = hi16 ? c0.odd : c0.even;
  const int p8 = hi16 ? c8.odd : c8.even;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      const bf16x4 lo = read_tr(t, p0 + G::off(32 * mt + 16 * s, 4 * dt));
      const bf16x4 hi = read_tr(t, p8 + G::off(32 * mt + 16 * s, 4 * dt));
      v.a[s][dt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// The A operands of accum32_rows for DP = 96 (rows 32mt .. 32mt+31 of tile t), read with the
// LDS transpose load in one asm block that waits for its own reads before it ends.  The
// builtin makes the compiler wait for every copy in flight first (it cannot tell LDS stages
// apart for this load); a caller of this version must itself make sure the tile has landed
// and that no copy in flight targets it.
__device__ inline void read_rows32_96(const RowTile<bf16, 96>& t, RowsFrag32<96>& v, int lane, int half, int mt) {
  using G = TileGeom<bf16, 96>;
  const int lane16 = lane & 15, hi16 = (lane >> 4) & 1;
  const ColumnBases c0 = column_bases<96>(4 * half, lane16), c8 = column_bases<96>(8 + 4 * half, lane16);
  const int p0 = (hi16 ? c0.odd : c0.even) + G::off(32 * mt, 0);
  const int p8 = (hi16 ? c8.odd : c8.even) + G::off(32 * mt, 0);
  const uint32_t a0 = (uint32_t)(uintptr_t)(const lds_bf16*)(t.x + p0);
  const uint32_t a8 = (uint32_t)(uintptr_t)(const lds_bf16*)(t.x + p8);
  // byte offsets: rows 16 s (s = 0, 1) and column blocks 32 dt (dt = 0, 1, 2): 2 (16 s 96 + 32 dt)
  v4i16 l00, h00, l01, h01, l02, h02, l10, h10, l11, h11, l12, h12;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\t"
      "ds_read_b64_tr_b16 %1, %13\n\t"
      "ds_read_b64_tr_b16 %2, %12 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:64\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:128\n\t"
      "ds_read_b64_tr_b16 %6, %12 offset:3072\n\t"
      "ds_read_b64_tr_b16 %7, %13 offset:3072\n\t"
      "ds_read_b64_tr_b16 %8, %12 offset:3136\n\t"
      "ds_read_b64_tr_b16 %9, %13 offset:3136\n\t"
      "ds_read_b64_tr_b16 %10, %12 offset:3200\n\t"
      "ds_read_b64_tr_b16 %11, %13 offset:3200\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l00), "=&v"(h00), "=&v"(l01), "=&v"(h01), "=&v"(l02), "=&v"(h02), "=&v"(l10), "=&v"(h10),
        "=&v"(l11), "=&v"(h11), "=&v"(l12), "=&v"(h12)
      : "v"(a0), "v"(a8)
      : "memory");
  const v4i16 lo[2][3] = {{l00, l01, l02}, {l10, l11, l12}};
  const v4i16 hi[2][3] = {{h00, h01, h02}, {h10, h11, h12}};
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      const bf16x4 l = __builtin_bit_cast(bf16x4, lo[s][dt]);
      const bf16x4 h = __builtin_bit_cast(bf16x4, hi[s][dt]);
      v.a[s][dt] = bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    }
}

// Rows 8(i/4) + 4h + i%4 of a 32x32 score block (slot i, lane half h) whose bit is clear in
// `mine` become -inf.
__device__ inline void mask_rows32(f32x16& s, uint32_t mine, int half) {
  const uint32_t mh = mine >> (4 * half);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (!((mh >> (8 * (i >> 2) + (i & 3))) & 1u)) s[i] = -INFINITY;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// p = exp2(c s - m) for the 16 slots of a 32x32 score block, rounded to bf16 into the B
// operand of accum32 (pb[s] holds slots 8s .. 8s+7).  Returns the sum of the rounded
// values (two per v_dot2 against (1, 1), fp32 accumulation): the weights the product
// with V actually uses.
__device__ inline float exp_pack32(const f32x16& s, float c, float m, bf16x8 (&pb)[2]) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x2 q = {(bf16)fast_exp2(fmaf(s[2 * j], c, -m)), (bf16)fast_exp2(fmaf(s[2 * j + 1], c, -m))};
    pb[j >> 2][2 * (j & 3)] = q[0];
    pb[j >> 2][2 * (j & 3) + 1] = q[1];
    sum = __builtin_amdgcn_fdot2_f32_bf16(q, one, sum, false);
  }
  return sum;
}

// acc[dt] += V^T P with the A operands read beforehand by read_rows32 and the B operand
// packed by exp_pack32.
template <int DP>
__device__ inline void accum32_packed(const RowsFrag32<DP>& v, const bf16x8 (&pb)[2], f32x16 (&acc)[DP / 32]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v.a[s][dt], pb[s], acc[dt], 0, 0, 0);
}

// ---- direct global -> LDS copies ------------------------------------------------------
// buffer_load_dwordx4 ... lds writes the 16 bytes lane l loads to LDS address
// M0 + 16 l (dword size: M0 + 4 l), and an out-of-range load writes zeros.  One wave
// instruction therefore fills 64 consecutive 16-byte slots of a tile: slot p of a
// RowTile holds row p / CH, stored chunk p % CH, i.e. logical chunk (p % CH) ^ swz(row),
// and each lane loads exactly that chunk.  No registers hold tile data, so the copies of
// later tiles stay in flight while the current one is used.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

// Wait until at most n vector-memory instructions of this wave are outstanding.
template <int n>
__device__ inline void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Barrier between the steps of a direct-copy pipeline, where waves only read LDS and
// copies are in flight.  No release fence: one would wait for every outstanding copy,
// later tiles' included.  The copies the next step needs are waited for explicitly
// (wait_vm) before it, this wave's LDS reads are complete (lgkmcnt(0)) so a stage can
// be overwritten once every wave has passed, and the acquire fence keeps later LDS
// reads below the barrier.
__device__ inline void barrier_copies() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DP, int NT>
struct TileDma {
  using G = TileGeom<bf16, DP>;
  static constexpr int CH = G::RS / 8;
  static_assert(G::RS == DP, "direct copies need unpadded rows");
  static_assert(kTile * CH % NT == 0, "tile slots must spread evenly over the threads");
  static constexpr int ROUNDS = kTile * CH / NT;  // vector-memory instructions per tile and wave
  int row[ROUNDS];   // tile row of this lane's slot in round i
  int loffb[ROUNDS]; // byte offset of that slot's logical chunk in a dense [64][DP] tile
  __device__ inline TileDma() {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int p = i * NT + (int)threadIdx.x;  // = (i * NT / 64 + wave) * 64 + lane
      const int r = p / CH, c = (p - r * CH) ^ G::swz(r);
      row[i] = r;
      loffb[i] = (r * DP + (c << 3)) * 2;
    }
  }
  __device__ static inline lds_void* dst(RowTile<bf16, DP>& t, int i, int w) {
    return (lds_void*)((lds_char*)t.x + (i * NT + 64 * w) * 16);
  }
  // Tile rows contiguous from element `base` of src (the same on every lane); all rows valid.
  // The uniform part of the address goes in the scalar offset, so a copy costs no vector
  // instruction besides itself.
  __device__ inline void issue_at(const Src& src, RowTile<bf16, DP>& t, uint32_t base) const {
    const int w = wave_id();
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base * 2u));
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, dst(t, i, w), 16, (uint32_t)loffb[i], b, 0, 0);
  }
  // Row r from element offset rowoff(r) of src (r < valid); rows past `valid` become zero.
  template <typename RowOff>
  __device__ inline void issue(const Src& src, RowTile<bf16, DP>& t, int valid, RowOff rowoff) const {
    const int w = wave_id();
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int r = row[i];
      const uint32_t off = r < valid ? (uint32_t)(rowoff(r) + (loffb[i] >> 1) - r * DP) * 2u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, dst(t, i, w), 16, off, 0, 0, 0);
    }
  }
};

template <int S> using Stage_ = std::integral_constant<int, S>;

// NS-stage pipeline over tiles 0 .. total-1 that arrive by direct LDS copies:
// issue(Stage_<s>{}, t) starts the copies of tile t into LDS stage s, and every wave
// issues exactly PER_TILE vector-memory instructions in it; compute(Stage_<s>{}, t) uses
// the tile.  Tile t lives in stage t % NS; stages are compile-time constants (the loop
// is unrolled NS times), so each stage can be its own LDS object, which lets the
// compiler see that reading one stage does not depend on copies into another.  Tile
// t + NS - 1 is issued right after the barrier that follows every wave's compute(t - 1),
// whose stage it reuses; tiles t+1 .. t+NS-2 stay in flight meanwhile.
template <int NS, int PER_TILE, int S, typename Issue, typename Compute>
__device__ inline void pipeline_step(int t, int total, Issue& issue, Compute& compute) {
  if (NS == 3 && t + 1 < total) wait_vm<PER_TILE>();
  else wait_vm<0>();
  barrier_copies();
  if (t + NS - 1 < total) issue(Stage_<(S + NS - 1) % NS>{}, t + NS - 1);
  compute(Stage_<S>{}, t);
}

template <int NS, int PER_TILE, typename Issue, typename Compute>
__device__ inline void pipeline_lds(int total, Issue issue, Compute compute) {
  static_assert(NS == 2 || NS == 3, "two or three stages");
  if (total > 0) issue(Stage_<0>{}, 0);
  if (NS == 3 && total > 1) issue(Stage_<1>{}, 1);
  for (int t = 0; t < total; t += NS) {
    pipeline_step<NS, PER_TILE, 0>(t, total, issue, compute);
    if (t + 1 < total) pipeline_step<NS, PER_TILE, 1>(t + 1, total, issue, compute);
    if constexpr (NS == 3)
      if (t + 2 < total) pipeline_step<NS, PER_TILE, 2>(t + 2, total, issue, compute);
  }
}

// Register-staged tile copies, for a software pipeline: fetch() issues every 16-byte
// global load of a tile at once (no dependency between them), store() writes them to
// LDS later, so the loads of a later tile are in flight while the current one is
// computed.
template <typename T, int DP, int NT = kThreads>
struct RowRegs {
  using G = TileGeom<T, DP>;
  static constexpr int V = G::vec;
  static constexpr int n = kTile * DP / V / NT;
  static_assert(kTile * DP / V % NT == 0, "tile chunks must spread evenly");
  uint4 r[n];
  // rowoff(r) = element offset of row r (r < valid); rows past `valid` read zero
  template <typename RowOff>
  __device__ inline void fetch(const Src& src, int valid, RowOff rowoff) {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * NT;
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
      const int c = threadIdx.x + i * NT;
      r[i] = src.load16(b + (uint32_t)c * (uint32_t)(V * sizeof(T)));  // row-major: chunk c at c * V
    }
  }
  __device__ inline void store(RowTile<T, DP>& t) const {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / (DP / V), ch = c - row * (DP / V);
      *(uint4*)&t.x[G::chunk(row, ch)] = r[i];
    }
  }
};

// Two-stage software pipeline over tiles 0 .. total-1: the global loads of tile t+2 are
// issued (into the stage tile t used) right after tile t is stored to LDS, so they have
// two tile computations to land.  fetch(stage, t) issues the loads, store(stage) writes
// the staged tile to LDS, compute(t) consumes it.  The loop is unrolled by two so each
// stage is a named register set (no dynamically indexed registers).
template <typename Stage, typename Fetch, typename Store, typename Compute>
__device__ inline void pipeline2(int total, Stage& s0, Stage& s1, Fetch fetch, Store store, Compute compute) {
  if (total > 0) fetch(s0, 0);
  if (total > 1) fetch(s1, 1);
  for (int t = 0; t < total; t += 2) {
    __syncthreads();  // the previous tile's readers are done with LDS
    store(s0);
    __syncthreads();
    if (t + 2 < total) fetch(s0, t + 2);
    compute(t);
    if (t + 1 < total) {
      __syncthreads();
      store(s1);
      __syncthreads();
      if (t + 3 < total) fetch(s1, t + 3);
      compute(t + 1);
    }
  }
}

// One-stage variant: the loads of tile t+1 are issued right after tile t is stored.
template <typename Stage, typename Fetch, typename Store, typename Compute>
__device__ inline void pipeline1(int total, Stage& s0, Fetch fetch, Store store, Compute compute) {
  if (total > 0) fetch(s0, 0);
  for (int t = 0; t < total; ++t) {
    __syncthreads();
    store(s0);
    __syncthreads();
    if (t + 1 < total) fetch(s0, t + 1);
    compute(t);
  }
}

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
};

// Bit r set: tile row r is a canonical slot that holds a token (occ: one bit per slot of
// the volume).  Lane r tests row r; every lane of the wave must call it.
__device__ inline uint64_t occupied_rows(const uint32_t* __restrict__ occ, const VirtualRows& vr, int valid) {
  const int lane = threadIdx.x & 63;
  bool p = false;
  if (lane < valid) {
    const int row = vr.row(lane);
    p = (occ[row >> 5] >> (row & 31)) & 1u;
  }
  return __ballot(p);
}

// Whether any of the n canonical rows from row0 holds a token.
__device__ inline bool any_occupied(const uint32_t* __restrict__ occ, int row0, int n) {
  const int lane = threadIdx.x & 63;
  bool p = false;
  for (int r = lane; r < n; r += 64) p |= (occ[(row0 + r) >> 5] >> ((row0 + r) & 31)) & 1u;
  return __ballot(p) != 0ull;
}

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
