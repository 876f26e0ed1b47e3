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
// goes through LDS.  K tiles [64 keys][Dp] and V^T tiles [Dp][64 keys] are staged
// in LDS; V is stored transposed inside each block by the RoPE kernel so the V^T
// tile rows are contiguous in HBM.
//   bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulation, fp32 softmax (exp2).
//   fp32: v_mfma_f32_16x16x4_f32 (full fp32 products).
// Local tiles come from the compacted neighbour list (a virtual concatenation of
// the neighbour blocks); summary tiles walk all block means in id order, masking
// the local blocks with an LDS bitmask, and tiles with no unmasked row are skipped.
// Deterministic: fixed reduction order, no atomics.
#include <cmath>

#include "tiles.h"

namespace pack3d {
namespace {

struct FwdArgs {
  const void* qrot; const void* krot; const void* vt; const void* kbar; const void* vbart;
  const int32_t* perm; const int32_t* nbr;
  void* out; float* lse;
  int N, H, D, nblk, nblkp, bvol, slots, tiles_per_block, with_summaries;
  float scale_log2;  // softmax scale * log2(e)
};

template <typename T, int DP>
struct FwdSmem {
  RowTile<T, DP> k;
  TrTile<T, DP> vt;
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  int nloc;
};

// Online-softmax state of one lane: query column (lane & 15).
template <int DP>
struct State {
  f32x4 o[DP / 16];
  float m, l;
};

// Scale, mask, online-softmax update and P.V for one staged tile.
// valid(r) says whether tile row r (0..63) is a real, unmasked key.
template <typename T, int DP, typename Valid>
__device__ inline void tile_step(const FwdSmem<T, DP>& sm, const ColFrag<T, DP>& f, State<DP>& st, float scale_log2,
                                 int col, int grp, Valid valid) {
  f32x4 s[4];
  score(sm.k, f, s, col, grp);
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = s[mt][i] * scale_log2;
      if (!valid(16 * mt + 4 * grp + i)) x = -INFINITY;
      s[mt][i] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  // m_new is finite: every query's first tile holds keys of its own block
  const float alpha = exp2f(st.m - m_new);
  st.m = m_new;
  float ls = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(s[mt][i] - m_new);
      s[mt][i] = p;
      ls += p;
    }
  }
  st.l = st.l * alpha + ls;
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) st.o[dt] *= alpha;
  accum(sm.vt, s, st.o, col, grp);
}

template <typename T, int DP>
__global__ __launch_bounds__(kThreads) void k_attn_fwd(FwdArgs a) {
  __shared__ FwdSmem<T, DP> sm;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int qb = tile / a.tiles_per_block, qsub = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int N = a.N, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nq = bvol < kTile ? bvol : kTile;
  const int qrow0 = qb * bvol + qsub * kTile;
  const int mask_words = a.nblkp / 32;

  // compacted neighbour list (wave 0) and the summary bitmask of the local blocks
  for (int i = tid; i < mask_words; i += kThreads) sm.mask[i] = 0u;
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

  // local stream: the neighbour blocks' keys as one virtual list of nloc * bvol rows
  const T* krot = (const T*)a.krot + bh * N * DP;
  const T* vt = (const T*)a.vt + bh * a.nblk * DP * bvol;
  const int nkeys = nloc * bvol;
  const int ntiles = (nkeys + kTile - 1) / kTile;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kTile;
    const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
    load_rows(sm.k, krot, valid, [&](int r) -> int64_t {
      const int j = j0 + r, blk = sm.list[j / bvol];
      return ((int64_t)blk * bvol + (j - (j / bvol) * bvol)) * DP;
    });
    load_tr(sm.vt, vt, valid, [&](int d, int r) -> int64_t {
      const int j = j0 + r, blk = sm.list[j / bvol];
      return ((int64_t)blk * DP + d) * bvol + (j - (j / bvol) * bvol);
    });
    __syncthreads();
    tile_step<T, DP>(sm, f, st, a.scale_log2, col, grp, [&](int r) { return r < valid; });
    __syncthreads();
  }

  // summary stream
  __syncthreads();  // the local-block bitmask is complete
  if (a.with_summaries) {
    const T* kbar = (const T*)a.kbar + bh * a.nblkp * DP;
    const T* vbart = (const T*)a.vbart + bh * DP * a.nblkp;
    const int nst = a.nblkp / kTile;
    for (int t = 0; t < nst; ++t) {
      const int r0 = t * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * t + 1] << 32) | sm.mask[2 * t];
      const uint64_t live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
      if (live == 0ull) continue;  // uniform: every row of this tile is local or padding
      load_rows(sm.k, kbar, kTile, [&](int r) -> int64_t { return (int64_t)(r0 + r) * DP; });
      load_tr(sm.vt, vbart, kTile, [&](int d, int r) -> int64_t { return (int64_t)d * a.nblkp + r0 + r; });
      __syncthreads();
      tile_step<T, DP>(sm, f, st, a.scale_log2, col, grp, [&](int r) { return ((live >> r) & 1ull) != 0ull; });
      __syncthreads();
    }
  }

  // epilogue: o = acc / l, lse = m ln2 + ln l, scattered back to packed order
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qloc < nq) {
    const int src = a.perm[(int64_t)b * N + qrow0 + qloc];
    const float inv = 1.0f / l;
    T* orow = (T*)a.out + (((int64_t)b * N + src) * a.H + h) * a.D;
#pragma unroll
    for (int dt = 0; dt < DP / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * dt + 4 * grp + i;
        if (d < a.D) orow[d] = (T)(st.o[dt][i] * inv);
      }
    }
    if (grp == 0) a.lse[bh * N + src] = st.m * kLn2 + logf(l);
  }
}

template <typename T>
pack3d_status launch_typed(const Dims& d, const FwdArgs& a, hipStream_t s) {
  dim3 grid(d.nblk * a.tiles_per_block, d.H, d.B);
  ProfileScope prof(a.with_summaries ? "attn_fwd" : "attn_fwd_windowed", s);
  switch (d.Dp) {
    case 32: hipLaunchKernelGGL((k_attn_fwd<T, 32>), grid, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_attn_fwd<T, 64>), grid, dim3(kThreads), 0, s, a); break;
    case 96: hipLaunchKernelGGL((k_attn_fwd<T, 96>), grid, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((k_attn_fwd<T, 128>), grid, dim3(kThreads), 0, s, a); break;
    default: return set_error(PACK3D_E_UNSUPPORTED, "forward: padded head dim %d", d.Dp);
  }
  return check_launch("forward: attention");
}

}  // namespace

pack3d_status launch_attn_fwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                              const char* ws, const Workspace& w, void* out, float* lse, hipStream_t s) {
  FwdArgs a;
  a.qrot = ws + w.qrot; a.krot = ws + w.krot; a.vt = ws + w.vt; a.kbar = ws + w.kbar; a.vbart = ws + w.vbart;
  a.perm = ix->perm; a.nbr = ix->nbr; a.out = out; a.lse = lse;
  a.N = d.N; a.H = d.H; a.D = d.D; a.nblk = d.nblk; a.nblkp = d.nblkp; a.bvol = d.bvol; a.slots = d.slots;
  a.tiles_per_block = d.bvol > kTile ? d.bvol / kTile : 1;
  a.with_summaries = at->with_summaries ? 1 : 0;
  const float scale = at->softmax_scale > 0.f ? at->softmax_scale : 1.0f / std::sqrt((float)d.D);
  a.scale_log2 = scale * kLog2e;
  return at->dtype == PACK3D_BF16 ? launch_typed<bf16>(d, a, s) : launch_typed<float>(d, a, s);
}

}  // namespace pack3d
