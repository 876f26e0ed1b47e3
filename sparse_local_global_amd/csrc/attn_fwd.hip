// K3: fused PACK3D attention forward (local key tiles, then summary tiles, one
// online softmax), hand-written for gfx950 matrix cores.
//
// "Geometry Matters in Packed 3D Attention" (abstract): local neighbourhood
// attention stays exact, distant context is compressed into contiguous 3D block
// summaries, and both kinds of logits share one softmax.  Reading: a query's local
// keys are every token of the blocks within Chebyshev distance r of its block (the
// neighbour table), its summaries are the block means of every other block of the
// volume; scale = 1/sqrt(D) unless given.
//
// Work decomposition: one workgroup (4 wave64s) per (64-query tile, head, volume).
// The tile's queries lie inside one block, so they share the key set.  Each wave
// owns 16 queries and keeps them in registers as the B operand of S^T = K Q^T, so
// the score tile comes out of the matrix core with one query per lane column; the
// softmax statistics of a query then live in 4 lanes (l, l^16, l^32, l^48) and the
// probabilities are already in the B-operand layout of O^T += V^T P^T, so P never
// goes through LDS.  K and V tiles [64 keys][Dp] are staged row-major in LDS; the
// P.V contraction reads V's columns with the LDS transpose load.
//   bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulation, fp32 softmax (exp2).
//   fp32: v_mfma_f32_16x16x4_f32 (full fp32 products).
// Local tiles come from the compacted neighbour list (a virtual concatenation of
// the neighbour blocks); summary tiles walk all block means in id order, masking
// the local blocks (and the padding rows) with an LDS bitmask.
// bf16 at Dp 32 and 96 (rows without padding) runs k_attn_fwd32d instead: four waves
// split into query halves and key halves with v_mfma_f32_32x32x16_bf16, tiles copied
// straight into LDS by buffer loads (no staging registers), the key halves' softmax
// states merged at the end; the other bf16 widths run the two-wave k_attn_fwd32.
// Deterministic: fixed reduction order, no atomics.
#include <cmath>

#include "tiles.h"

namespace pack3d {
namespace {

// NC canonical rows per volume; Nmax: lse stride; holes: canonical slots may be empty
// (occ: bit per slot, emask: bit per empty block), else both are unused.
struct FwdArgs {
  const void* qrot; const void* krot; const void* vr; const void* kbar; const void* vbar;
  const int32_t* perm; const int32_t* nbr; const int32_t* voff;
  const uint32_t* occ; const uint32_t* emask;
  void* out; float* lse;
  int NC, Nmax, H, D, nblk, nblkp, bvol, slots, tiles_per_block, with_summaries, holes, occ_words;
  float scale_log2;  // softmax scale * log2(e)
};

template <typename T, int DP>
struct FwdSmem {
  RowTile<T, DP> k;
  RowTile<T, DP> v;
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  int nloc;
};

// Online-softmax state of one lane: query column (lane & 15).  m is the running
// reference maximum in log2 units of the scaled logits.
template <int DP>
struct State {
  f32x4 o[DP / 16];
  float m, l;
};

// Rescaling is lazy: the reference maximum moves only when a tile's maximum exceeds it
// by more than kRescale (log2 units), so probabilities stay below 2^kRescale and most
// tiles skip the accumulator rescale.  The result is exact up to rounding for any
// reference, since numerator and denominator share it.
constexpr float kRescale = 8.0f;
// The same bound as a sum of weights (the bf16 kernels test sums, not maxima).
constexpr float kSumLimit = 256.0f;

// One staged tile: scores, mask, online-softmax update and P.V.  Bit r of `live` says
// whether tile row r is a real, unmasked key; all-ones tiles skip the masking.
template <typename T, int DP>
__device__ inline void tile_step(const FwdSmem<T, DP>& sm, const ColFrag<T, DP>& f, State<DP>& st, float c,
                                 int col, int grp, uint64_t live) {
  f32x4 s[4];
  score(sm.k, f, s, col, grp);
  if (live != ~0ull) {
    const uint64_t bits = live >> (4 * grp);  // row 16mt + 4grp + i -> bit 16mt + i
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t w = (uint32_t)(bits >> (16 * mt));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((w >> i) & 1u)) s[mt][i] = -INFINITY;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                       fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  mx *= c;  // scale > 0: the maximum of the scaled logits
  if (mx > st.m + kRescale) {
    // tiles without a live row are skipped, so mx is finite here
    const float alpha = fast_exp2(st.m - mx);
    st.m = mx;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DP / 16; ++dt) st.o[dt] *= alpha;
  }
  const float mneg = -st.m;
  float ls = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(fmaf(s[mt][i], c, mneg));
      s[mt][i] = p;
      ls += p;
    }
  }
  st.l += ls;
  accum(sm.v, s, st.o, col, grp);
}

// ONE_BLOCK: |b| is a multiple of 64, so every 64-row tile lies inside one block.
template <typename T, int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_attn_fwd(FwdArgs a) {
  __shared__ FwdSmem<T, DP> sm;
  // 1-D grid over (tile, head, volume), tile fastest, remapped so each XCD walks neighbouring tiles
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int qb = tile / a.tiles_per_block, qsub = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nq = bvol < kTile ? bvol : kTile;
  const int qrow0 = qb * bvol + qsub * kTile;
  const int mask_words = a.nblkp / 32;
  const uint32_t* occ = a.occ + (int64_t)b * a.occ_words;
  if (a.holes && !any_occupied(occ, qrow0, nq)) return;  // no token among the tile's queries

  // compacted neighbour list (wave 0) and the summary bitmask: empty blocks start
  // masked, the local blocks are added below
  for (int i = tid; i < mask_words; i += kThreads) sm.mask[i] = a.holes ? a.emask[(int64_t)b * mask_words + i] : 0u;
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + qb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = sm.nloc;
  for (int i = tid; i < nloc; i += kThreads) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));

  const int qloc = 16 * wave + col;
  ColFrag<T, DP> f;
  f.load((const T*)a.qrot + (bh * N + qrow0 + qloc) * DP, qloc < nq, grp);
  State<DP> st;
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;

  // Tile sequence: the local stream (the neighbour blocks' keys as one virtual list of
  // nloc * bvol rows) then the summary stream (all block means, local ones masked).
  // Software pipeline: the global loads of tile t+1 are issued before tile t is computed.
  const size_t es = sizeof(T);
  const Src krot((const T*)a.krot + bh * N * DP, (size_t)N * DP * es);
  const Src vrow((const T*)a.vr + bh * N * DP, (size_t)N * DP * es);
  const Src kbar((const T*)a.kbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const Src vbar((const T*)a.vbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const int nkeys = nloc * bvol;
  const int nlt = (nkeys + kTile - 1) / kTile;
  const int total = nlt + (a.with_summaries ? a.nblkp / kTile : 0);
  // two register stages: the loads of tile t+2 are issued while tile t is computed
  struct Stage {
    RowRegs<T, DP> k, v;
  } st0, st1;
  const int tpk = bvol / kTile;  // tiles per block (ONE_BLOCK)
  auto fetch = [&](Stage& S, int t) {
    if (t < nlt) {
      if constexpr (ONE_BLOCK) {
        const int q = t / tpk, off = (t - q * tpk) * kTile;
        const int blk = sm.list[q];
        S.k.fetch_at(krot, (uint32_t)(blk * bvol + off) * DP);
        S.v.fetch_at(vrow, (uint32_t)(blk * bvol + off) * DP);
      } else {
        const int j0 = t * kTile;
        const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
        const VirtualRows vr(sm.list, bvol, j0);
        S.k.fetch(krot, valid, [&](int r) { return vr.row(r) * DP; });
        S.v.fetch(vrow, valid, [&](int r) { return vr.row(r) * DP; });
      }
    } else {
      const int r0 = (t - nlt) * kTile;
      S.k.fetch_at(kbar, (uint32_t)r0 * DP);
      S.v.fetch_at(vbar, (uint32_t)r0 * DP);
    }
  };
  auto store = [&](const Stage& S) {
    S.k.store(sm.k);
    S.v.store(sm.v);
  };
  auto compute = [&](int t) {
    uint64_t live;
    if (t < nlt) {
      const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
      live = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
      if (a.holes) live &= occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
    } else {
      const int ts = t - nlt, r0 = ts * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * ts + 1] << 32) | sm.mask[2 * ts];
      live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
    }
    if (live == 0ull) return;  // all masked (empty slots): nothing to add, and m may still be -inf
    tile_step(sm, f, st, c, col, grp, live);
  };
  pipeline2(total, st0, st1, fetch, store, compute);

  // epilogue: o = acc / l, lse = m ln2 + ln l, scattered back to packed order
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int src = qloc < nq ? a.perm[(int64_t)b * N + qrow0 + qloc] : -1;  // -1: empty slot
  if (src >= 0) {
    const float inv = 1.0f / l;
    T* orow = (T*)a.out + (((int64_t)a.voff[b] + src) * a.H + h) * a.D;
#pragma unroll
    for (int dt = 0; dt < DP / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * dt + 4 * grp + i;
        if (d < a.D) orow[d] = (T)(st.o[dt][i] * inv);
      }
    }
    if (grp == 0) a.lse[bh * a.Nmax + src] = st.m * kLn2 + logf(l);
  }
}

// ---- bf16: two wave64s per 64-query tile, 32 query columns per wave ------------------
// v_mfma_f32_32x32x16_bf16 reads each 16-byte K / V fragment from LDS once per 32
// query columns (half the LDS traffic per multiply of the 16-column layout), and the
// row maximum of a query needs one cross-lane step (lanes l and l ^ 32).
constexpr int kThreads32 = 128;

template <int DP>
struct State32 {
  f32x16 o[DP / 32];
  float m, l;
};

template <int DP>
__device__ inline void tile_step32(const FwdSmem<bf16, DP>& sm, const ColFrag32<DP>& f, State32<DP>& st, float c,
                                   int lane, int half, uint64_t live) {
  const int col = lane & 31;
  f32x16 s[2];
  score32(sm.k, f, s, col, half);
  if (live != ~0ull) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mt + 8 * (i >> 2) + 4 * half + (i & 3);
        if (!((live >> r) & 1ull)) s[mt][i] = -INFINITY;
      }
    }
  }
  float m0 = s[0][0], m1 = s[1][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    m0 = fmaxf(m0, s[0][i]);
    m1 = fmaxf(m1, s[1][i]);
  }
  float mx = fmaxf(m0, m1);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  mx *= c;  // scale > 0: the maximum of the scaled logits
  if (mx > st.m + kRescale) {
    const float alpha = fast_exp2(st.m - mx);
    st.m = mx;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) st.o[dt] *= alpha;
  }
  const float mneg = -st.m;
  float ls = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[mt][i], c, mneg));
      s[mt][i] = p;
      ls += p;
    }
  }
  st.l += ls;
  accum32(sm.v, s, st.o, lane, half);
}

template <int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads32) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_fwd32(FwdArgs a) {
  __shared__ FwdSmem<bf16, DP> sm;
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int qb = tile / a.tiles_per_block, qsub = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nq = bvol < kTile ? bvol : kTile;
  const int qrow0 = qb * bvol + qsub * kTile;
  const int mask_words = a.nblkp / 32;
  const uint32_t* occ = a.occ + (int64_t)b * a.occ_words;
  if (a.holes && !any_occupied(occ, qrow0, nq)) return;  // no token among the tile's queries

  for (int i = tid; i < mask_words; i += kThreads32) sm.mask[i] = a.holes ? a.emask[(int64_t)b * mask_words + i] : 0u;
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + qb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = sm.nloc;
  for (int i = tid; i < nloc; i += kThreads32) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));

  const int qloc = 32 * wave + col;
  ColFrag32<DP> f;
  f.load((const bf16*)a.qrot + (bh * N + qrow0 + qloc) * DP, qloc < nq, half);
  State32<DP> st;
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;

  const size_t es = sizeof(bf16);
  const Src krot((const bf16*)a.krot + bh * N * DP, (size_t)N * DP * es);
  const Src vrow((const bf16*)a.vr + bh * N * DP, (size_t)N * DP * es);
  const Src kbar((const bf16*)a.kbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const Src vbar((const bf16*)a.vbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const int nkeys = nloc * bvol;
  const int nlt = (nkeys + kTile - 1) / kTile;
  const int total = nlt + (a.with_summaries ? a.nblkp / kTile : 0);
  struct Stage {
    RowRegs<bf16, DP, kThreads32> k, v;
  } st0;
  const int tpk = bvol / kTile;
  auto fetch = [&](Stage& S, int t) {
    if (t < nlt) {
      if constexpr (ONE_BLOCK) {
        const int q = t / tpk, off = (t - q * tpk) * kTile;
        const int blk = sm.list[q];
        S.k.fetch_at(krot, (uint32_t)(blk * bvol + off) * DP);
        S.v.fetch_at(vrow, (uint32_t)(blk * bvol + off) * DP);
      } else {
        const int j0 = t * kTile;
        const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
        const VirtualRows vr(sm.list, bvol, j0);
        S.k.fetch(krot, valid, [&](int r) { return vr.row(r) * DP; });
        S.v.fetch(vrow, valid, [&](int r) { return vr.row(r) * DP; });
      }
    } else {
      const int r0 = (t - nlt) * kTile;
      S.k.fetch_at(kbar, (uint32_t)r0 * DP);
      S.v.fetch_at(vbar, (uint32_t)r0 * DP);
    }
  };
  auto store = [&](const Stage& S) {
    S.k.store(sm.k);
    S.v.store(sm.v);
  };
  auto compute = [&](int t) {
    uint64_t live;
    if (t < nlt) {
      const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
      live = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
      if (a.holes) live &= occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
    } else {
      const int ts = t - nlt, r0 = ts * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * ts + 1] << 32) | sm.mask[2 * ts];
      live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
    }
    if (live == 0ull) return;
    tile_step32(sm, f, st, c, lane, half, live);
  };
  pipeline1(total, st0, fetch, store, compute);

  // epilogue: o = acc / l, lse = m ln2 + ln l, scattered back to packed order
  float l = st.l + __shfl_xor(st.l, 32);
  const int src = qloc < nq ? a.perm[(int64_t)b * N + qrow0 + qloc] : -1;  // -1: empty slot
  if (src >= 0) {
    const float inv = 1.0f / l;
    bf16* orow = (bf16*)a.out + (((int64_t)a.voff[b] + src) * a.H + h) * a.D;
    if (a.D == DP) {
      // slots 4j .. 4j+3 are consecutive dims: 8-byte stores
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(bf16x4*)(orow + 32 * dt + 8 * j + 4 * half) =
              bf16x4{(bf16)(st.o[dt][4 * j] * inv), (bf16)(st.o[dt][4 * j + 1] * inv),
                     (bf16)(st.o[dt][4 * j + 2] * inv), (bf16)(st.o[dt][4 * j + 3] * inv)};
    } else {
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * dt + 8 * (i >> 2) + 4 * half + (i & 3);
          if (d < a.D) orow[d] = (bf16)(st.o[dt][i] * inv);
        }
      }
    }
    if (half == 0) a.lse[bh * a.Nmax + src] = st.m * kLn2 + logf(l);
  }
}

// ---- bf16 with direct LDS copies: four wave64s per 64-query tile ----------------------
// Waves (qh, kh): queries 32qh .. 32qh+31 against key rows 32kh .. 32kh+31 of every tile.
// The two key halves of a query keep independent online softmax states over disjoint key
// sets, merged at the end (max of the references, each side rescaled by exp2 of its
// distance to it): the same sums in another grouping.  Tiles arrive by buffer loads that
// write LDS directly (no staging registers, no LDS store instructions), two stages deep.
template <int DP>
struct FwdStage32 {
  RowTile<bf16, DP> k, v;
};

// Local key tiles whose live-row masks k_attn_fwd32d reads into LDS before its loop when
// slots can be empty (small enough to keep three workgroups per CU).
constexpr int kFwdLiveTiles = 32;

struct FwdSmem32d {
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  uint64_t live[kFwdLiveTiles];  // local tile t: bit r = key row r holds a token (empty slots only)
  int nloc;
};

// Two LDS stages (52 KB) leave room for three workgroups per CU, so three waves per SIMD.
template <int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void k_attn_fwd32d(FwdArgs a) {
  __shared__ FwdSmem32d sm;
  __shared__ FwdStage32<DP> s0, s1;
  static_assert(sizeof(f32x4) * (4 * DP / 32) * 64 * 2 <= sizeof(FwdStage32<DP>), "partial outputs fit a stage");
  static_assert(sizeof(float2) * 64 * 2 <= sizeof(FwdStage32<DP>), "partial statistics fit a stage");
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int qb = tile / a.tiles_per_block, qsub = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nq = bvol < kTile ? bvol : kTile;
  const int qrow0 = qb * bvol + qsub * kTile;
  const int mask_words = a.nblkp / 32;
  const uint32_t* occ = a.occ + (int64_t)b * a.occ_words;
  if (a.holes && !any_occupied(occ, qrow0, nq)) return;  // no token among the tile's queries

  // summary bitmask: empty blocks start masked, the local blocks are added below
  for (int i = tid; i < mask_words; i += kThreads) sm.mask[i] = a.holes ? a.emask[(int64_t)b * mask_words + i] : 0u;
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + qb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  // uniform by construction; readfirstlane lets the compiler keep the tile branches and
  // the buffer resources they select scalar
  const int nloc = __builtin_amdgcn_readfirstlane(sm.nloc);
  for (int i = tid; i < nloc; i += kThreads) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));

  const int qloc = 32 * qh + col;
  ColFrag32<DP> f;
  f.load((const bf16*)a.qrot + (bh * N + qrow0 + qloc) * DP, qloc < nq, half);
  // the query rows are in registers before any tile copy starts: otherwise the waits for
  // them at their first use inside the loop also wait for the copies in flight
  wait_vm<0>();
  State32<DP> st;
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;

  const size_t es = sizeof(bf16);
  const Src krot((const bf16*)a.krot + bh * N * DP, (size_t)N * DP * es);
  const Src vrow((const bf16*)a.vr + bh * N * DP, (size_t)N * DP * es);
  const Src kbar((const bf16*)a.kbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const Src vbar((const bf16*)a.vbar + bh * a.nblkp * DP, (size_t)a.nblkp * DP * es);
  const int nkeys = nloc * bvol;
  const int nlt = (nkeys + kTile - 1) / kTile;
  const int total = nlt + (a.with_summaries ? a.nblkp / kTile : 0);
  using Dma = TileDma<DP, kThreads>;
  const Dma dma;
  auto stage = [&](auto sg) -> FwdStage32<DP>& {
    if constexpr (decltype(sg)::value == 0) return s0;
    else return s1;
  };
  // (each instantiation of this generic lambda calls only one of issue_at and issue: with
  // both, the host compilation has left out launch stubs, see the explicit instantiations
  // in attn_bwd.hip)
  const bf16* kq = (const bf16*)a.krot + bh * N * DP;
  const bf16* vq = (const bf16*)a.vr + bh * N * DP;
  const bf16* kbq = (const bf16*)a.kbar + bh * a.nblkp * DP;
  const bf16* vbq = (const bf16*)a.vbar + bh * a.nblkp * DP;
  const size_t bytes_loc = (size_t)N * DP * es, bytes_sum = (size_t)a.nblkp * DP * es;
  // ONE_BLOCK: tiles are issued in order, so a cursor (entry of the neighbour list,
  // 64-row tile within that block) replaces a division per tile
  const int tpb = a.tiles_per_block;
  int cur_entry = 0, cur_sub = 0;
  auto issue = [&](auto sg, int t) {
    FwdStage32<DP>& S = stage(sg);
    if constexpr (ONE_BLOCK) {
      // one contiguous run per tensor: select the (uniform) base pointers and build the
      // buffer resources at one call site, so they stay scalar
      const bool loc = t < nlt;
      uint32_t row0 = (uint32_t)(t - nlt) * kTile;
      if (loc) {
        const int blk = __builtin_amdgcn_readfirstlane(sm.list[cur_entry]);
        row0 = (uint32_t)(blk * bvol + cur_sub * kTile);
        if (++cur_sub == tpb) {
          cur_sub = 0;
          ++cur_entry;
        }
      }
      const size_t bytes = loc ? bytes_loc : bytes_sum;
      const Src ks(loc ? kq : kbq, bytes), vs(loc ? vq : vbq, bytes);
      dma.issue_at(ks, S.k, row0 * DP);
      dma.issue_at(vs, S.v, row0 * DP);
      return;
    }
    if (t < nlt) {
      const int j0 = t * kTile;
      const VirtualRows vr(sm.list, bvol, j0);
      if constexpr (!ONE_BLOCK) {
        const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
        dma.issue(krot, S.k, valid, [&](int r) { return vr.row(r) * DP; });
        dma.issue(vrow, S.v, valid, [&](int r) { return vr.row(r) * DP; });
      }
    } else {
      const int r0 = (t - nlt) * kTile;
      dma.issue(kbar, S.k, kTile, [&](int r) { return (r0 + r) * DP; });
      dma.issue(vbar, S.v, kTile, [&](int r) { return (r0 + r) * DP; });
    }
  };
  // This wave's live key rows of tile t (bit r: row 32kh + r).  It runs before the next
  // tile's copies are issued: with empty slots it loads occupancy words, and a wait for
  // those would otherwise also wait for the copies.
  // With empty slots the local tiles' occupancy comes from global memory.  Up to
  // kFwdLiveTiles tiles it is read here, before the loop, one tile per wave at a time: in
  // the loop each such load would hold up its step for a whole memory latency.  The first
  // step's barrier orders these LDS writes before their reads.
  const bool live_table = a.holes && nlt <= kFwdLiveTiles;
  if (live_table) {
    for (int t = wave; t < nlt; t += kThreads / 64) {
      const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
      const uint64_t lv = occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
      if (lane == 0) sm.live[t] = lv;
    }
  }
  auto tile_occupancy = [&](int t, int valid) -> uint64_t {
    return live_table ? sm.live[t] : occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
  };
  auto live_rows = [&](int t) -> uint32_t {
    uint64_t live;
    if (t < nlt) {
      if constexpr (ONE_BLOCK) {
        live = a.holes ? tile_occupancy(t, kTile) : ~0ull;
      } else {
        const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
        live = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
        if (a.holes) live &= tile_occupancy(t, valid);
      }
    } else {
      const int ts = t - nlt, r0 = ts * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * ts + 1] << 32) | sm.mask[2 * ts];
      live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
    }
    // uniform, so the branches on it stay scalar
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(kh ? (uint32_t)(live >> 32) : (uint32_t)live));
  };
  // tile t with this wave's live rows `mine` (not zero)
  auto compute = [&](auto sg, uint32_t mine, const RowsFrag32<DP>& vfr) {
    const FwdStage32<DP>& S = stage(sg);
    f32x16 sc;
    // the K reads run three ahead of their products (more would spill at three waves per SIMD)
    score32_rows_ahead<DP, 3>(S.k, f, sc, col, half, kh);
    if (mine != ~0u) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * half + (i & 3);
        if (!((mine >> r) & 1u)) sc[i] = -INFINITY;
      }
    }
    // Exponentiate against the current reference maximum without looking for the tile's
    // own: when no lane's sum over its 16 keys exceeds kSumLimit, no weight exceeds it
    // either and the reference may stay (lazy rescaling, exact up to rounding since
    // numerator and denominator share it).  Otherwise, and on the first live tile where
    // no reference exists yet, the exact tile maximum becomes the reference.
    bf16x8 pb[2];
    float ls = 0.f;
    bool slow = __ballot(st.m == -INFINITY) != 0ull;
    if (!slow) {
      ls = exp_pack32(sc, c, st.m, pb);
      slow = __ballot(!(ls <= kSumLimit)) != 0ull;
    }
    if (slow) {
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= c;
      if (mx > st.m) {
        const float alpha = fast_exp2(st.m - mx);  // 0 while the reference is -inf (o, l are 0)
        st.m = mx;
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DP / 32; ++dt) st.o[dt] *= alpha;
      }
      ls = exp_pack32(sc, c, st.m, pb);
    }
    st.l += ls;
    accum32_packed(vfr, pb, st.o);
  };
  // Two stages.  The compiler makes every LDS transpose load wait for all copies in
  // flight, so each step reads its V operands right after the wait for its own tile and
  // only then starts the copies of the next tile into the stage the barrier freed; those
  // have the rest of the step to land.
  auto step = [&](auto sg, int t) {
    constexpr int SI = decltype(sg)::value;
    wait_vm<0>();
    barrier_copies();  // tile t is in stage SI; every wave is done with the other stage
    const uint32_t mine = live_rows(t);  // zero: nothing live here, and m may still be -inf
    RowsFrag32<DP> vfr;
    if (mine) read_rows32(stage(sg).v, vfr, lane, half, kh);
    if (t + 1 < total) issue(Stage_<1 - SI>{}, t + 1);
    if (mine) compute(sg, mine, vfr);
  };
  if (total > 0) issue(Stage_<0>{}, 0);
  for (int t = 0; t < total; t += 2) {
    step(Stage_<0>{}, t);
    if (t + 1 < total) step(Stage_<1>{}, t + 1);
  }
  __syncthreads();  // the stages are reused for the merge below

  // merge the key halves: waves kh = 1 leave (m, l, o) in stage 0 ([slot][lane] float4s)
  // and stage 1 (m, l per lane); waves kh = 0 combine and write the output
  f32x4* po = (f32x4*)&s0 + qh * (4 * DP / 32) * 64;
  float2* pml = (float2*)&s1 + qh * 64;
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        po[(4 * dt + q) * 64 + lane] = f32x4{st.o[dt][4 * q], st.o[dt][4 * q + 1], st.o[dt][4 * q + 2], st.o[dt][4 * q + 3]};
    pml[lane] = make_float2(st.m, st.l);
  }
  __syncthreads();
  if (kh == 1) return;
  const float2 ml = pml[lane];
  const float m = fmaxf(st.m, ml.x);
  // a side that saw no live key has m = -inf, l = 0, o = 0 and weight exp2(-inf) = 0
  const float w0 = st.m == -INFINITY ? 0.f : fast_exp2(st.m - m);
  const float w1 = ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - m);
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 o1 = po[(4 * dt + q) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) st.o[dt][4 * q + e] = st.o[dt][4 * q + e] * w0 + o1[e] * w1;
    }
  float l = st.l * w0 + ml.y * w1;
  l += __shfl_xor(l, 32);
  const int src = qloc < nq ? a.perm[(int64_t)b * N + qrow0 + qloc] : -1;  // -1: empty slot
  if (src >= 0) {
    const float inv = 1.0f / l;
    bf16* orow = (bf16*)a.out + (((int64_t)a.voff[b] + src) * a.H + h) * a.D;
    if (a.D == DP) {
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(bf16x4*)(orow + 32 * dt + 8 * j + 4 * half) =
              bf16x4{(bf16)(st.o[dt][4 * j] * inv), (bf16)(st.o[dt][4 * j + 1] * inv),
                     (bf16)(st.o[dt][4 * j + 2] * inv), (bf16)(st.o[dt][4 * j + 3] * inv)};
    } else {
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * dt + 8 * (i >> 2) + 4 * half + (i & 3);
          if (d < a.D) orow[d] = (bf16)(st.o[dt][i] * inv);
        }
      }
    }
    if (half == 0) a.lse[bh * a.Nmax + src] = m * kLn2 + logf(l);
  }
}

template <typename T, int DP>
void launch_dp(const Dims& d, const FwdArgs& a, dim3 grid, hipStream_t s) {
  // bf16 rows without padding in LDS (Dp 32, 96): four waves, direct LDS copies
  if constexpr (sizeof(T) == 2 && (DP == 32 || DP == 96)) {
    if (d.bvol % kTile == 0) hipLaunchKernelGGL((k_attn_fwd32d<DP, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_fwd32d<DP, false>), grid, dim3(kThreads), 0, s, a);
  } else if constexpr (sizeof(T) == 2 && DP <= 96) {
    // 32-column waves for the other bf16 widths up to Dp = 96 (at Dp = 128 their registers would spill)
    if (d.bvol % kTile == 0) hipLaunchKernelGGL((k_attn_fwd32<DP, true>), grid, dim3(kThreads32), 0, s, a);
    else hipLaunchKernelGGL((k_attn_fwd32<DP, false>), grid, dim3(kThreads32), 0, s, a);
  } else {
    if (d.bvol % kTile == 0) hipLaunchKernelGGL((k_attn_fwd<T, DP, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_fwd<T, DP, false>), grid, dim3(kThreads), 0, s, a);
  }
}

template <typename T>
pack3d_status launch_typed(const Dims& d, const FwdArgs& a, hipStream_t s) {
  dim3 grid(d.nblk * a.tiles_per_block * d.H * d.B);
  ProfileScope prof(a.with_summaries ? "attn_fwd" : "attn_fwd_windowed", s);
  switch (d.Dp) {
    case 32: launch_dp<T, 32>(d, a, grid, s); break;
    case 64: launch_dp<T, 64>(d, a, grid, s); break;
    case 96: launch_dp<T, 96>(d, a, grid, s); break;
    case 128: launch_dp<T, 128>(d, a, grid, s); break;
    default: return set_error(PACK3D_E_UNSUPPORTED, "forward: padded head dim %d", d.Dp);
  }
  return check_launch("forward: attention");
}

}  // namespace

pack3d_status launch_attn_fwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                              const char* ws, const Workspace& w, void* out, float* lse, hipStream_t s) {
  FwdArgs a;
  a.qrot = ws + w.qrot; a.krot = ws + w.krot; a.vr = ws + w.vr; a.kbar = ws + w.kbar; a.vbar = ws + w.vbar;
  a.perm = ix->perm; a.nbr = ix->nbr; a.voff = ix->voff; a.occ = ix->occ; a.emask = ix->emask;
  a.out = out; a.lse = lse;
  a.NC = d.NC; a.Nmax = d.Nmax; a.holes = d.holes; a.occ_words = ix->occ_words; a.H = d.H; a.D = d.D; a.nblk = d.nblk; a.nblkp = d.nblkp; a.bvol = d.bvol; a.slots = d.slots;
  a.tiles_per_block = d.bvol > kTile ? d.bvol / kTile : 1;
  a.with_summaries = at->with_summaries ? 1 : 0;
  const float scale = at->softmax_scale > 0.f ? at->softmax_scale : 1.0f / std::sqrt((float)d.D);
  a.scale_log2 = scale * kLog2e;
  return at->dtype == PACK3D_BF16 ? launch_typed<bf16>(d, a, s) : launch_typed<float>(d, a, s);
}

}  // namespace pack3d
