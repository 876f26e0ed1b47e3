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

#include "layout.h"

namespace pack3d {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct FwdArgs {
  const void* qrot; const void* krot; const void* vt; const void* kbar; const void* vbart;
  const int32_t* perm; const int32_t* nbr;
  void* out; float* lse;
  int N, H, D, nblk, nblkp, bvol, slots, tiles_per_block, with_summaries;
  float scale_log2;  // softmax scale * log2(e)
};

template <typename T> struct Mma;

// bf16: K rows padded by 8 elements, V^T rows by 8 (16-byte aligned rows).
template <> struct Mma<bf16> {
  static constexpr int kPad = 8, vPad = 8;
  static constexpr int kVec = 8;   // elements per 16-byte global load
};
template <> struct Mma<float> {
  static constexpr int kPad = 4, vPad = 4;
  static constexpr int kVec = 4;
};

template <typename T, int DP>
struct alignas(16) Smem {
  T k[kTile][DP + Mma<T>::kPad];
  T v[DP][kTile + Mma<T>::vPad];
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  int nloc;
};

// Cooperative 16-byte copies of one K tile and one V^T tile into LDS.
// key_base(j8) returns the element offset of key row j (local: gathered through the
// neighbour list; summaries: contiguous), vt_base(d, j8) the offset of 8 (or 4)
// consecutive keys of V^T row d.  Rows past `valid` are zero-filled.
template <typename T, int DP, typename KRow, typename VRow>
__device__ inline void load_tile(Smem<T, DP>& sm, const T* __restrict__ kg, const T* __restrict__ vg, int valid,
                                 KRow krow, VRow vrow) {
  constexpr int V = Mma<T>::kVec;
  constexpr int kchunks = kTile * DP / V;
  for (int c = threadIdx.x; c < kchunks; c += kThreads) {
    const int row = c / (DP / V), cc = (c - row * (DP / V)) * V;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (row < valid) x = *(const uint4*)(kg + krow(row) + cc);
    *(uint4*)&sm.k[row][cc] = x;
  }
  constexpr int vchunks = DP * kTile / V;
  for (int c = threadIdx.x; c < vchunks; c += kThreads) {
    const int d = c / (kTile / V), j = (c - d * (kTile / V)) * V;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (j < valid) x = *(const uint4*)(vg + vrow(d, j));
    *(uint4*)&sm.v[d][j] = x;
  }
}

// Online-softmax state of one lane: query column (lane & 15), 4 row groups.
template <int DP>
struct State {
  f32x4 o[DP / 16];
  float m, l;
};

template <typename T, int DP>
struct Frag;

template <int DP>
struct Frag<bf16, DP> {
  bf16x8 q[DP / 32];
  __device__ inline void load(const bf16* __restrict__ row, bool ok, int grp) {
#pragma unroll
    for (int s = 0; s < DP / 32; ++s) {
      if (ok) q[s] = *(const bf16x8*)(row + 32 * s + 8 * grp);
      else q[s] = bf16x8{};
    }
  }
  __device__ inline void scores(const Smem<bf16, DP>& sm, f32x4 (&s)[4], int col, int grp) const {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DP / 32; ++k) {
        const bf16x8 a = *(const bf16x8*)&sm.k[16 * mt + col][32 * k + 8 * grp];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q[k], acc, 0, 0, 0);
      }
      s[mt] = acc;
    }
  }
  // O^T[d][q] += sum_key V^T[d][key] P^T[key][q]; k slot e of lane group g holds key
  // 32c + 4g + e (e < 4) or 32c + 16 + 4g + (e - 4) (e >= 4), in both operands.
  __device__ inline void pv(const Smem<bf16, DP>& sm, const f32x4 (&p)[4], f32x4 (&o)[DP / 16], int col, int grp) const {
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
        const bf16x4 lo = *(const bf16x4*)&sm.v[16 * dt + col][32 * c + 4 * grp];
        const bf16x4 hi = *(const bf16x4*)&sm.v[16 * dt + col][32 * c + 16 + 4 * grp];
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[dt], 0, 0, 0);
      }
    }
  }
};

template <int DP>
struct Frag<float, DP> {
  // lane group g holds head dims [g*DP/4, (g+1)*DP/4) of its query
  float q[DP / 4];
  __device__ inline void load(const float* __restrict__ row, bool ok, int grp) {
#pragma unroll
    for (int s = 0; s < DP / 4; s += 4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (ok) x = *(const f32x4*)(row + grp * (DP / 4) + s);
      q[s] = x[0]; q[s + 1] = x[1]; q[s + 2] = x[2]; q[s + 3] = x[3];
    }
  }
  __device__ inline void scores(const Smem<float, DP>& sm, f32x4 (&s)[4], int col, int grp) const {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DP / 4; k += 4) {
        const f32x4 a = *(const f32x4*)&sm.k[16 * mt + col][grp * (DP / 4) + k];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], q[k + e], acc, 0, 0, 0);
      }
      s[mt] = acc;
    }
  }
  // k index g of MFMA (mt, i) is key 16mt + 4g + i in both operands.
  __device__ inline void pv(const Smem<float, DP>& sm, const f32x4 (&p)[4], f32x4 (&o)[DP / 16], int col, int grp) const {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int dt = 0; dt < DP / 16; ++dt) {
        const f32x4 a = *(const f32x4*)&sm.v[16 * dt + col][16 * mt + 4 * grp];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], p[mt][i], o[dt], 0, 0, 0);
      }
    }
  }
};

// Scale, mask, online-softmax update and P.V for one staged tile.
// valid(r) says whether tile row r (0..63) is a real, unmasked key.
template <typename T, int DP, typename Valid>
__device__ inline void tile_step(const Smem<T, DP>& sm, const Frag<T, DP>& f, State<DP>& st, float scale_log2,
                                 int col, int grp, Valid valid) {
  f32x4 s[4];
  f.scores(sm, s, col, grp);
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
  f.pv(sm, s, st.o, col, grp);
}

template <typename T, int DP>
__global__ __launch_bounds__(kThreads) void k_attn_fwd(FwdArgs a) {
  __shared__ Smem<T, DP> sm;
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
  if (wave == 0) {
    int base = 0;
    const int32_t* nb = a.nbr + ((int64_t)b * a.nblk + qb) * a.slots;
    for (int c = 0; c < a.slots; c += 64) {
      const int s = c + lane;
      const int id = s < a.slots ? nb[s] : -1;
      const uint64_t m = __ballot(id >= 0);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (id >= 0) sm.list[pos] = id;
      base += __popcll(m);
    }
    if (lane == 0) sm.nloc = base;
  }
  __syncthreads();
  const int nloc = sm.nloc;
  for (int i = tid; i < nloc; i += kThreads) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));

  const int qloc = 16 * wave + col;
  Frag<T, DP> f;
  f.load((const T*)a.qrot + (bh * N + qrow0 + qloc) * DP, qloc < nq, grp);
  State<DP> st;
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  // local stream
  const T* krot = (const T*)a.krot + bh * N * DP;
  const T* vt = (const T*)a.vt + bh * a.nblk * DP * bvol;
  const int nkeys = nloc * bvol;
  const int ntiles = (nkeys + kTile - 1) / kTile;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kTile;
    const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
    load_tile<T, DP>(sm, krot, vt, valid,
        [&](int r) -> int64_t {
          const int j = j0 + r, blk = sm.list[j / bvol];
          return ((int64_t)blk * bvol + (j - (j / bvol) * bvol)) * DP;
        },
        [&](int d, int r) -> int64_t {
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
      const uint32_t w0 = sm.mask[2 * t], w1 = sm.mask[2 * t + 1];
      const uint64_t used = ((uint64_t)w1 << 32) | w0;
      const uint64_t live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
      if (live == 0ull) continue;  // uniform: every row of this tile is local or padding
      load_tile<T, DP>(sm, kbar, vbart, kTile,
          [&](int r) -> int64_t { return (int64_t)(r0 + r) * DP; },
          [&](int d, int r) -> int64_t { return (int64_t)d * a.nblkp + r0 + r; });
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
