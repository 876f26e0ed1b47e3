// PACK3D backward: gradients of sum(out * dout) with respect to the unrotated q, k, v,
// through the shared softmax, the block mean pooling and the axial RoPE.
//
// "Geometry Matters in Packed 3D Attention" (abstract) presents the operator as
// trainable at scale; the gradients follow from its definition.  With
// P = exp(logit - lse) for local keys j and summaries b of query i,
//   delta_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, V_j> - delta_i),  dT_ib = P_ib (<dO_i, Vbar_b> - delta_i)
//   dQ~_i   = scale (sum_j dS_ij K~_j + sum_b dT_ib Kbar_b)
//   dK~_j   = scale sum_i dS_ij Q~_i + dKbar_b(j) / n_b,  dKbar_b = scale sum_i dT_ib Q~_i
//   dV_j    = sum_i P_ij dO_i + dVbar_b(j) / n_b,         dVbar_b = sum_i P_ib dO_i
//   dq = R(c)^T dQ~, dk = R(c)^T dK~  (R orthogonal; the mean broadcasts 1/n_b to each of
//   the n_b tokens present in block b, n_b = |b| on a full grid).
// Empty canonical slots (ragged geometry) hold zero rows of Q~, K~, V and dO, and lse
// +inf, so they add nothing to any sum; the query-major dQ kernel masks them as keys,
// as the forward does, and no kernel writes a gradient for them.
//
// Kernels, in launch order (no atomics anywhere, so results are bitwise reproducible):
//   bwd_pre      per block: -delta, dO and lse (in log2 units) gathered to canonical order
//   bwd_summary  summary-major: each workgroup owns 64 summaries of one (volume, head) and a
//                chunk of query blocks; masks the summaries local to each query block and
//                accumulates partial dKbar, dVbar (fp32) per chunk
//   bwd_reduce   sums the chunks in a fixed order
//   bwd_local    key-major: each workgroup owns 64 keys and walks the query tiles of their
//                neighbour blocks (the neighbourhood is symmetric) for dK~, dV; the epilogue
//                adds the broadcast summary gradients, applies R^T and scatters dk, dv to
//                packed order
//   bwd_dq       query-major (like the forward, recomputing P from lse): dQ~ over local and
//                summary tiles; the epilogue applies R^T and scatters dq
// The waves hold their 16 columns (keys, summaries or queries) in registers and stream
// row-major 64-row tiles through LDS; the two contraction shapes are the ones of
// tiles.h (the accumulate shape reads tile columns with the LDS transpose load).
#include <cmath>

#include "tiles.h"

namespace pack3d {
namespace {

struct BwdArgs {
  // forward intermediates and backward layouts (workspace, canonical order)
  const void* qrot; const void* krot; const void* vr; const void* kbar; const void* vbar;
  // lsec: lse * log2(e); ndelta: -<dO, O> (score products of dP accumulate onto it); canonical order
  void* doc; float* lsec; float* ndelta;
  float* dkbar; float* dvbar; float* part_k; float* part_v;
  const float2* tab;
  // caller buffers (packed order)
  const void* out; const float* lse; const void* dout;
  void* dq; void* dk; void* dv;
  const int32_t* coords; const int32_t* perm; const int32_t* nbr; const int32_t* geom;
  const int32_t* voff; const int32_t* count; const uint32_t* occ; const uint32_t* emask;
  // NC canonical rows per volume, Nmax the lse stride, holes: empty slots exist
  int B, NC, Nmax, H, D, Dp, nblk, nblkp, bvol, slots, radius, tiles_per_block, with_summaries, chunks;
  int holes, occ_words;
  int64_t grad_stride;  // elements between consecutive tokens of dq, dk, dv
  int pos_mode, groups, gw, half, trows;  // rotation groups (see Dims)
  int bz, by, bx;
  float scale, scale_log2;
};

template <typename T, int V>
struct alignas(sizeof(T) * V) Vec {
  T v[V];
};

// 1 / n_b of block kb of volume b: the tokens present (|b| on a full grid); 0 for an
// empty block, whose gradients are never written.
__device__ inline float block_inv(const BwdArgs& a, int b, int kb) {
  const int cnt = a.holes ? a.count[(int64_t)b * a.nblk + kb] : a.bvol;
  return cnt > 0 ? 1.0f / (float)cnt : 0.f;
}

// ---------------------------------------------------------------------------------
// bwd_pre: one workgroup per (block, head, volume)
// ---------------------------------------------------------------------------------
template <typename T, int VEC>
__global__ __launch_bounds__(256) void k_bwd_pre(BwdArgs a) {
  extern __shared__ char smem[];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int N = a.NC, D = a.D, Dp = a.Dp, bvol = a.bvol;
  const int ntok = bvol < kTile ? bvol : kTile;
  const int nch = D / VEC;
  float* part = (float*)smem;                          // [ntok][nch] partial dot products
  const int64_t bh = (int64_t)b * a.H + h;
  const T* dout = (const T*)a.dout;
  const T* out = (const T*)a.out;
  T* doc = (T*)a.doc;
  for (int t0 = 0; t0 < bvol; t0 += ntok) {
    for (int it = tid; it < ntok * nch; it += 256) {
      const int tok = it / nch, c = (it - tok * nch) * VEC;
      const int kappa = blk * bvol + t0 + tok;
      const int src = a.perm[(int64_t)b * N + kappa];   // -1: empty slot, zero row
      Vec<T, VEC> g, o;
      if (src >= 0) {
        const int64_t in = (((int64_t)a.voff[b] + src) * a.H + h) * D + c;
        g = *(const Vec<T, VEC>*)(dout + in);
        o = *(const Vec<T, VEC>*)(out + in);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) g.v[e] = o.v[e] = (T)0.f;
      }
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += (float)g.v[e] * (float)o.v[e];
      part[it] = acc;   // it = tok * nch + chunk index
      *(Vec<T, VEC>*)(doc + (bh * N + kappa) * Dp + c) = g;
    }
    if (Dp > D) {
      const int pad = Dp - D;
      for (int it = tid; it < ntok * pad; it += 256) {
        const int tok = it / pad, c = D + it - tok * pad;
        doc[(bh * N + blk * bvol + t0 + tok) * Dp + c] = (T)0.f;
      }
    }
    __syncthreads();
    if (tid < ntok) {
      const int kappa = blk * bvol + t0 + tid;
      const int src = a.perm[(int64_t)b * N + kappa];
      float s = 0.f;
      for (int c = 0; c < nch; ++c) s += part[tid * nch + c];
      a.ndelta[bh * N + kappa] = -s;
      // log2 units; +inf for an empty slot makes every probability of that row 0
      a.lsec[bh * N + kappa] = src >= 0 ? a.lse[bh * a.Nmax + src] * kLog2e : INFINITY;
    }
    __syncthreads();
  }
}

// The same for bf16 rows without padding with every head in one workgroup: the workgroup
// takes TPW consecutive canonical slots, and its items run over (slot, head, 8-element piece)
// with the piece fastest, so consecutive threads read consecutive 16 bytes of a token's dO
// and O rows (H * D contiguous elements each).  Each thread loads all three of its items
// before it stores any.  The sums run in the same order as in k_bwd_pre (each piece, then
// the pieces of a row in order), so the results are bitwise the same.
constexpr int kPreItems = 3;  // items per thread

__global__ __launch_bounds__(256) void k_bwd_pre_rows(BwdArgs a, int tpw) {
  constexpr int VEC = 8;
  extern __shared__ char smem[];
  float* part = (float*)smem;  // [tpw][H][nch] piece dot products
  const int H = a.H, D = a.D, N = a.NC, nch = D / VEC;
  const int per_slot = H * nch;
  const int tid = threadIdx.x, b = blockIdx.y;
  const int kappa0 = blockIdx.x * tpw;
  const int64_t tok0 = a.voff[b];
  Vec<bf16, VEC> g[kPreItems], o[kPreItems];
#pragma unroll
  for (int u = 0; u < kPreItems; ++u) {
    const int it = tid + 256 * u, q = it / per_slot, rem = it - q * per_slot;
    const int h = rem / nch, c = rem - h * nch;
    const int kappa = kappa0 + q;
    const int src = q < tpw && kappa < N ? a.perm[(int64_t)b * N + kappa] : -1;
    if (src >= 0) {
      const int64_t in = ((tok0 + src) * H + h) * D + c * VEC;
      g[u] = *(const Vec<bf16, VEC>*)((const bf16*)a.dout + in);
      o[u] = *(const Vec<bf16, VEC>*)((const bf16*)a.out + in);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[u].v[e] = o[u].v[e] = (bf16)0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < kPreItems; ++u) {
    const int it = tid + 256 * u, q = it / per_slot, rem = it - q * per_slot;
    const int h = rem / nch, c = rem - h * nch;
    const int kappa = kappa0 + q;
    if (q >= tpw || kappa >= N) continue;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += (float)g[u].v[e] * (float)o[u].v[e];
    part[it] = acc;
    *(Vec<bf16, VEC>*)((bf16*)a.doc + (((int64_t)b * H + h) * N + kappa) * D + c * VEC) = g[u];
  }
  __syncthreads();
  if (tid < tpw * H) {
    const int q = tid / H, h = tid - q * H, kappa = kappa0 + q;
    if (kappa < N) {
      const int64_t bh = (int64_t)b * H + h;
      const int src = a.perm[(int64_t)b * N + kappa];
      float s = 0.f;
      for (int c = 0; c < nch; ++c) s += part[(q * H + h) * nch + c];
      a.ndelta[bh * N + kappa] = -s;
      // log2 units; +inf for an empty slot makes every probability of that row 0
      a.lsec[bh * N + kappa] = src >= 0 ? a.lse[bh * a.Nmax + src] * kLog2e : INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------------
// Epilogue shared by bwd_local and bwd_dq: rows of fp32 gradients staged in LDS
// (canonical rows row0 .. row0+nrows), optionally rotated back by R^T, written in
// the output dtype to packed order.
// ---------------------------------------------------------------------------------
template <typename T>
__device__ inline void write_rows(const BwdArgs& a, const float* st, int sts, int nrows, int b, int h, int row0,
                                  bool unrotate, T* dst, int* s_src, int* s_rel) {
  const int tid = threadIdx.x;
  const int N = a.NC, D = a.D;
  const int64_t tok0 = a.voff[b];
  if (tid < nrows) {
    const int src = a.perm[(int64_t)b * N + row0 + tid];   // -1: empty slot, not written
    s_src[tid] = src;
    const int32_t* g = a.geom + b * G_FIELDS;
    const int32_t* c = a.coords + (tok0 + (src >= 0 ? src : 0)) * 3;
    for (int gi = 0; gi < a.groups; ++gi) s_rel[tid * 3 + gi] = rope_row(a.pos_mode, gi, src, c, g, a.trows);
  }
  __syncthreads();
  const int gw = a.gw, half = a.half;
  unrotate = unrotate && a.pos_mode != PACK3D_POS_NONE;
  for (int it = tid; it < nrows * D; it += (int)blockDim.x) {
    const int r = it / D, col = it - r * D;
    if (s_src[r] < 0) continue;
    float v = st[r * sts + col];
    if (unrotate) {
      const int ax = col / gw, k = col - ax * gw;
      const int kk = k < half ? k : k - half;
      const float2 cs = a.tab[(int64_t)s_rel[r * 3 + ax] * half + kk];
      if (k < half) v = v * cs.x + st[r * sts + col + half] * cs.y;      // y1 c + y2 s
      else v = -st[r * sts + col - half] * cs.y + v * cs.x;              // -y1 s + y2 c
    }
    dst[(tok0 + s_src[r]) * a.grad_stride + (int64_t)h * D + col] = (T)v;
  }
  __syncthreads();  // s_src / s_rel are rewritten by the next call
}

// ---------------------------------------------------------------------------------
// bwd_summary: workgroup = (64 summaries, head, volume x query chunk).  Wide fp32 rows
// (Dp >= 64) run one wave per SIMD so the accumulators can use the AGPRs instead of
// spilling; bwd_local below does the same.
// ---------------------------------------------------------------------------------
template <typename T, int DP>
struct SumSmem {
  RowTile<T, DP> q, g;
  float lse[kTile], ndelta[kTile];
};

template <typename T, int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DP * sizeof(T) <= 192 ? 2 : 1, 2)))
void k_bwd_summary(BwdArgs a) {
  __shared__ SumSmem<T, DP> sm;
  // 1-D grid over (summary tile, chunk, head, volume), summary tile fastest: the
  // workgroups that share a chunk's query tiles run on the same XCD
  const int nst = a.nblkp / kTile;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int r0 = (L % nst) * kTile, chunk = (L / nst) % a.chunks;
  const int h = (L / nst / a.chunks) % a.H, b = L / nst / a.chunks / a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int sid = r0 + 16 * wave + col;          // this lane's summary (block id)
  ColFrag<T, DP> kf, vf;
  kf.load((const T*)a.kbar + (bh * a.nblkp + sid) * DP, true, grp);   // padding rows are zero
  vf.load((const T*)a.vbar + (bh * a.nblkp + sid) * DP, true, grp);
  const int32_t* g = a.geom + b * G_FIELDS;
  // the volume's block grid covers its bounding box: ceil(extent / b) blocks per axis
  const int nby = (g[G_EY] + a.by - 1) / a.by, nbx = (g[G_EX] + a.bx - 1) / a.bx;
  const int sz = sid / (nby * nbx), sy = (sid / nbx) % nby, sx = sid % nbx;
  f32x4 dk[DP / 16], dv[DP / 16];
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int q_begin = (int)((int64_t)chunk * a.nblk / a.chunks);
  const int q_end = (int)((int64_t)(chunk + 1) * a.nblk / a.chunks);
  const int nrow = bvol < kTile ? bvol : kTile;
  const int tpb = a.tiles_per_block;
  const size_t slice = (size_t)N * DP * sizeof(T);
  const Src qrot((const T*)a.qrot + bh * N * DP, slice);
  const Src doc((const T*)a.doc + bh * N * DP, slice);
  const float c = a.scale_log2;
  // tile t = (query block q_begin + t / tpb, sub-tile t % tpb); pipelined like the forward
  const int total = (q_end - q_begin) * tpb;
  struct Stage {
    RowRegs<T, DP> q, g;
    float lse2, ndelta;  // of tile row tid (tid < 64)
  } st0, st1;
  auto fetch = [&](Stage& S, int t) {
    const int qb = q_begin + t / tpb, qs = t - (t / tpb) * tpb;
    const int row0 = qb * bvol + qs * kTile;
    if constexpr (ONE_BLOCK) {
      S.q.fetch_at(qrot, (uint32_t)row0 * DP);
      S.g.fetch_at(doc, (uint32_t)row0 * DP);
    } else {
      S.q.fetch(qrot, nrow, [&](int r) { return (row0 + r) * DP; });
      S.g.fetch(doc, nrow, [&](int r) { return (row0 + r) * DP; });
    }
    if (tid < kTile) {
      S.lse2 = tid < nrow ? a.lsec[bh * N + row0 + tid] : INFINITY;
      S.ndelta = tid < nrow ? a.ndelta[bh * N + row0 + tid] : 0.f;
    }
  };
  auto store = [&](const Stage& S) {
    S.q.store(sm.q);
    S.g.store(sm.g);
    if (tid < kTile) {
      sm.lse[tid] = S.lse2;
      sm.ndelta[tid] = S.ndelta;
    }
  };
  auto compute = [&](int t) {
    const int qb = q_begin + t / tpb;
    const int qz = qb / (nby * nbx), qy = (qb / nbx) % nby, qx = qb % nbx;
    const int cheb = max(max(abs(qz - sz), abs(qy - sy)), abs(qx - sx));
    const bool masked = sid >= a.nblk || cheb <= a.radius;
    f32x4 s[4], dp[4];
    score(sm.q, kf, s, col, grp);
    // dp = <dO, V> - delta: the products accumulate onto -delta of rows 16mt + 4grp + i
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dp[mt] = *(const f32x4*)&sm.ndelta[16 * mt + 4 * grp];
    score_acc(sm.g, vf, dp, col, grp);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * grp + i;
        float p = fast_exp2(fmaf(s[mt][i], c, -sm.lse[r]));
        if (masked) p = 0.f;
        s[mt][i] = p;
        dp[mt][i] = p * dp[mt][i];
      }
    }
    accum(sm.g, s, dv, col, grp);
    accum(sm.q, dp, dk, col, grp);
  };
  pipeline2(total, st0, st1, fetch, store, compute);
  const int64_t base = (((int64_t)chunk * a.B * a.H + bh) * a.nblkp + sid) * DP;
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) {
    *(f32x4*)(a.part_k + base + 16 * dt + 4 * grp) = dk[dt] * a.scale;
    *(f32x4*)(a.part_v + base + 16 * dt + 4 * grp) = dv[dt];
  }
}

__global__ void k_bwd_reduce(const float* __restrict__ pk, const float* __restrict__ pv, float* dk, float* dv,
                             int64_t n, int chunks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < chunks; ++c) {
    sk += pk[c * n + i];
    sv += pv[c * n + i];
  }
  dk[i] = sk;
  dv[i] = sv;
}

// ---------------------------------------------------------------------------------
// bwd_local: workgroup = (64 keys of one block, head, volume)
// ---------------------------------------------------------------------------------
template <typename T, int DP>
struct LocSmem {
  union {
    struct {
      RowTile<T, DP> q, g;
    } t;
    float st[kTile][DP + 1];
  } u;
  float lse[kTile], ndelta[kTile];
  int list[kMaxSlots];
  int nloc;
  int src[kTile], rel[kTile * 3];
};

template <typename T, int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DP * sizeof(T) <= 192 ? 2 : 1, 2)))
void k_bwd_local(BwdArgs a) {
  __shared__ LocSmem<T, DP> sm;
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int kb = tile / a.tiles_per_block, ks = tile - kb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nk = bvol < kTile ? bvol : kTile;
  const int krow0 = kb * bvol + ks * kTile;
  if (a.holes && !any_occupied(a.occ + (int64_t)b * a.occ_words, krow0, nk)) return;  // no key here
  const int kloc = 16 * wave + col;
  ColFrag<T, DP> kf, vf;
  kf.load((const T*)a.krot + (bh * N + krow0 + kloc) * DP, kloc < nk, grp);
  vf.load((const T*)a.vr + (bh * N + krow0 + kloc) * DP, kloc < nk, grp);
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + kb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = sm.nloc;
  f32x4 dk[DP / 16], dv[DP / 16];
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t slice = (size_t)N * DP * sizeof(T);
  const Src qrot((const T*)a.qrot + bh * N * DP, slice);
  const Src doc((const T*)a.doc + bh * N * DP, slice);
  const float c = a.scale_log2;
  const int nq = nloc * bvol;
  const int ntiles = (nq + kTile - 1) / kTile;
  struct Stage {
    RowRegs<T, DP> q, g;
    float lse2, ndelta;  // of tile row tid (tid < 64)
  } st0, st1;
  auto fetch = [&](Stage& S, int t) {
    const int j0 = t * kTile;
    const int valid = nq - j0 < kTile ? nq - j0 : kTile;
    const VirtualRows vr(sm.list, bvol, j0);
    if constexpr (ONE_BLOCK) {
      const int row0 = vr.blk0 * bvol + vr.off0;
      S.q.fetch_at(qrot, (uint32_t)row0 * DP);
      S.g.fetch_at(doc, (uint32_t)row0 * DP);
    } else {
      S.q.fetch(qrot, valid, [&](int r) { return vr.row(r) * DP; });
      S.g.fetch(doc, valid, [&](int r) { return vr.row(r) * DP; });
    }
    if (tid < kTile) {
      S.lse2 = INFINITY;   // padding rows: P = 0
      S.ndelta = 0.f;
      if (tid < valid) {
        const int row = vr.row(tid);
        S.lse2 = a.lsec[bh * N + row];
        S.ndelta = a.ndelta[bh * N + row];
      }
    }
  };
  auto store = [&](const Stage& S) {
    S.q.store(sm.u.t.q);
    S.g.store(sm.u.t.g);
    if (tid < kTile) {
      sm.lse[tid] = S.lse2;
      sm.ndelta[tid] = S.ndelta;
    }
  };
  auto compute = [&](int) {
    f32x4 s[4], dp[4];
    score(sm.u.t.q, kf, s, col, grp);
    // dp = <dO, V> - delta: the products accumulate onto -delta of rows 16mt + 4grp + i
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) dp[mt] = *(const f32x4*)&sm.ndelta[16 * mt + 4 * grp];
    score_acc(sm.u.t.g, vf, dp, col, grp);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * grp + i;
        const float p = fast_exp2(fmaf(s[mt][i], c, -sm.lse[r]));   // lse = +inf -> 0
        s[mt][i] = p;
        dp[mt][i] = p * dp[mt][i];
      }
    }
    accum(sm.u.t.g, s, dv, col, grp);
    accum(sm.u.t.q, dp, dk, col, grp);
  };
  pipeline2(ntiles, st0, st1, fetch, store, compute);
  __syncthreads();  // the staging area below overlays the tiles

  // epilogue: dK~ = scale * acc + dKbar / |b| (then R^T), dV = acc + dVbar / |b|, each
  // staged through the same LDS rows and scattered to packed order
  const float inv = block_inv(a, b, kb);
  const float* dkb = a.dkbar + (bh * a.nblkp + kb) * DP;
  const float* dvb = a.dvbar + (bh * a.nblkp + kb) * DP;
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * dt + 4 * grp + i;
      sm.u.st[kloc][d] = dk[dt][i] * a.scale + (a.with_summaries ? dkb[d] * inv : 0.f);
    }
  }
  __syncthreads();
  write_rows<T>(a, &sm.u.st[0][0], DP + 1, nk, b, h, krow0, true, (T*)a.dk, sm.src, sm.rel);
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * dt + 4 * grp + i;
      sm.u.st[kloc][d] = dv[dt][i] + (a.with_summaries ? dvb[d] * inv : 0.f);
    }
  }
  __syncthreads();
  write_rows<T>(a, &sm.u.st[0][0], DP + 1, nk, b, h, krow0, false, (T*)a.dv, sm.src, sm.rel);
}

// ---------------------------------------------------------------------------------
// bwd_local for bf16 with 32 key columns per wave, fed by direct LDS copies.
// Workgroup = (64 keys, head, volume) as above, four waves: key half kh = wave & 1 and
// query-row half qh = wave >> 1 of every query tile; the two query halves' partial
// dK~, dV are summed through LDS before the epilogue.  v_mfma_f32_32x32x16_bf16 halves
// the LDS reads per multiply against 16-column waves, and the copies (query tile, dO
// tile, lse, -delta) hold no registers, so three LDS stages keep two tiles in flight.
// Rows past the end of the last tile arrive as zeros: Q = dO = 0 there, so their
// probabilities multiply zero rows and add nothing.
// ---------------------------------------------------------------------------------
constexpr int kLdsStages = 3;

template <int DP>
struct LocStage32 {
  RowTile<bf16, DP> q, g;
  float lse2[kTile], ndelta[kTile];
};

template <int DP>
struct LocSmem32 {
  int list[kMaxSlots];
  int nloc;
  int src[kTile], rel[kTile * 3];
};

// Epilogue of bwd_local32 for D = 96, in registers.  Each RoPE axis is then exactly
// one 32-dim accumulator block (dt = axis) and the pair (k, k + 16) of a rotation sits in
// slots i and i + 8 of the same lane, so R^T needs no data exchange.  The two query
// halves swap partial sums through LDS (half 1 sends dK~, half 0 sends dV); half 0 then
// finishes dk = R^T (scale * acc + dKbar / |b|), half 1 dv = acc + dVbar / |b|, and each
// lane stores its key's 48 values as 8-byte pieces.
__device__ inline void local32_epilogue96(const BwdArgs& a, f32x16 (&dk)[3], f32x16 (&dv)[3], f32x4* part, int b,
                                          int h, int kb, int krow0, int kloc, int nk, int qh, int lane, int half) {
  constexpr int NDT = 3;
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[(4 * dt + q) * 64 + lane] = f32x4{dk[dt][4 * q], dk[dt][4 * q + 1], dk[dt][4 * q + 2], dk[dt][4 * q + 3]};
  } else {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[(4 * NDT + 4 * dt + q) * 64 + lane] =
            f32x4{dv[dt][4 * q], dv[dt][4 * q + 1], dv[dt][4 * q + 2], dv[dt][4 * q + 3]};
  }
  __syncthreads();
  const int64_t bh = (int64_t)b * a.H + h;
  const float inv = block_inv(a, b, kb);
  f32x16(&acc)[NDT] = dk;  // the half's own tensor; filled below for qh = 1
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = dv[dt];
  }
  const int pslot = qh == 0 ? 0 : 4 * NDT;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 pv = part[(pslot + 4 * dt + q) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[dt][4 * q + e] += pv[e];
    }
  if (kloc >= nk) return;
  const float* sb = (qh == 0 ? a.dkbar : a.dvbar) + (bh * a.nblkp + kb) * 96;
  const float mul = qh == 0 ? a.scale : 1.0f;
  // value of dim 32dt + 8jj + 4half + e is slot 4jj + e of block dt
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 sv = a.with_summaries ? *(const f32x4*)(sb + 32 * dt + 8 * jj + 4 * half) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[dt][4 * jj + e] = acc[dt][4 * jj + e] * mul + sv[e] * inv;
    }
  const int row = krow0 + kloc;
  const int src = a.perm[(int64_t)b * a.NC + row];
  if (src < 0) return;  // empty slot
  const int64_t tok0 = a.voff[b];
  // R^T on the lane's own pairs: every pair partner (+16 within an axis group, +48 for the
  // 1D rotation) keeps the dim's residue mod 8, so it sits in the same lane
  if (qh == 0 && a.pos_mode == PACK3D_POS_AXIAL) {
    const int32_t* g = a.geom + b * G_FIELDS;
    const int32_t* c = a.coords + (tok0 + src) * 3;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      int r = c[dt] - g[G_OZ + dt];
      r = r < 0 ? 0 : (r >= a.trows ? a.trows - 1 : r);
      const float2* cs = a.tab + (int64_t)r * 16 + 4 * half;  // half = 16 pairs per axis
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 t = cs[8 * j + e];
          const float lo = acc[dt][4 * j + e], hi = acc[dt][4 * j + 8 + e];
          acc[dt][4 * j + e] = lo * t.x + hi * t.y;       // y1 c + y2 s
          acc[dt][4 * j + 8 + e] = -lo * t.y + hi * t.x;  // -y1 s + y2 c
        }
    }
  } else if (qh == 0 && a.pos_mode == PACK3D_POS_PACKED_1D) {
    const float2* cs = a.tab + (int64_t)src * 48 + 4 * half;  // 48 pairs (k, k + 48) per row
#pragma unroll
    for (int m = 0; m < 6; ++m)  // dims 8m + 4 half + e and 8(m + 6) + 4 half + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 t = cs[8 * m + e];
        const float y1 = acc[m / 4][4 * (m % 4) + e], y2 = acc[(m + 6) / 4][4 * ((m + 6) % 4) + e];
        acc[m / 4][4 * (m % 4) + e] = y1 * t.x + y2 * t.y;
        acc[(m + 6) / 4][4 * ((m + 6) % 4) + e] = -y1 * t.y + y2 * t.x;
      }
  }
  bf16* dst = (bf16*)(qh == 0 ? a.dk : a.dv) + (tok0 + src) * a.grad_stride + (int64_t)h * 96;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *(bf16x4*)(dst + 32 * dt + 8 * jj + 4 * half) =
          bf16x4{(bf16)acc[dt][4 * jj], (bf16)acc[dt][4 * jj + 1], (bf16)acc[dt][4 * jj + 2], (bf16)acc[dt][4 * jj + 3]};
}

// Direct copy of lse2 / -delta for tile rows 16 w .. 16 w + 15 (lanes 0..15 of wave w).
__device__ inline void issue_rows16(const Src& src, float* dst16, uint32_t byte_off) {
  if ((threadIdx.x & 63) < 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (lds_void*)dst16, 4, byte_off, 0, 0, 0);
}

template <int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_local32(BwdArgs a) {
  __shared__ LocSmem32<DP> sm;
  // one LDS object per stage; the epilogue reuses them: query half 1's partial dK~, dV
  // for key half 0 / 1 in stages 0 / 1 ([slot][lane] float4s), the staging rows in stage 2
  __shared__ LocStage32<DP> s0, s1, s2;
  static_assert(sizeof(f32x4) * DP / 32 * 8 * 64 <= sizeof(LocStage32<DP>), "partials fit a stage");
  static_assert(sizeof(float) * kTile * (DP + 1) <= sizeof(LocStage32<DP>), "staging rows fit a stage");
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int kb = tile / a.tiles_per_block, ks = tile - kb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nk = bvol < kTile ? bvol : kTile;
  const int krow0 = kb * bvol + ks * kTile;
  if (a.holes && !any_occupied(a.occ + (int64_t)b * a.occ_words, krow0, nk)) return;  // no key here
  const int kloc = 32 * kh + col;
  ColFrag32<DP> kf, vf;
  kf.load((const bf16*)a.krot + (bh * N + krow0 + kloc) * DP, kloc < nk, half);
  vf.load((const bf16*)a.vr + (bh * N + krow0 + kloc) * DP, kloc < nk, half);
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + kb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = sm.nloc;
  f32x16 dk[DP / 32], dv[DP / 32];
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) dk[dt] = dv[dt] = f32x16{};

  const size_t slice = (size_t)N * DP * sizeof(bf16);
  const Src qrot((const bf16*)a.qrot + bh * N * DP, slice);
  const Src doc((const bf16*)a.doc + bh * N * DP, slice);
  const Src lsec(a.lsec + bh * N, (size_t)N * sizeof(float));
  const Src dlt(a.ndelta + bh * N, (size_t)N * sizeof(float));
  const float c = a.scale_log2;
  const int nq = nloc * bvol;
  const int ntiles = (nq + kTile - 1) / kTile;
  using Dma = TileDma<DP, kThreads>;
  const Dma dma;
  auto stage = [&](auto st) -> LocStage32<DP>& {
    if constexpr (decltype(st)::value == 0) return s0;
    else if constexpr (decltype(st)::value == 1) return s1;
    else return s2;
  };
  // ONE_BLOCK: tiles are issued in order, so a cursor (entry of the neighbour list, 64-row
  // tile within that block) replaces a division per tile
  const int tpb = a.tiles_per_block;
  int cur_entry = 0, cur_sub = 0;
  auto issue = [&](auto st, int t) {
    LocStage32<DP>& S = stage(st);
    const int j0 = t * kTile;
    const int w = wave_id(), r = 16 * w + (lane & 15);
    if constexpr (ONE_BLOCK) {
      const int row0 = __builtin_amdgcn_readfirstlane(sm.list[cur_entry]) * bvol + cur_sub * kTile;
      if (++cur_sub == tpb) {
        cur_sub = 0;
        ++cur_entry;
      }
      dma.issue_at(qrot, S.q, (uint32_t)row0 * DP);
      dma.issue_at(doc, S.g, (uint32_t)row0 * DP);
      issue_rows16(lsec, &S.lse2[16 * w], (uint32_t)(row0 + r) * 4u);
      issue_rows16(dlt, &S.ndelta[16 * w], (uint32_t)(row0 + r) * 4u);
    } else {
      const VirtualRows vr(sm.list, bvol, j0);
      const int valid = nq - j0 < kTile ? nq - j0 : kTile;
      dma.issue(qrot, S.q, valid, [&](int rr) { return vr.row(rr) * DP; });
      dma.issue(doc, S.g, valid, [&](int rr) { return vr.row(rr) * DP; });
      const uint32_t off = r < valid ? (uint32_t)vr.row(r) * 4u : 0x80000000u;
      issue_rows16(lsec, &S.lse2[16 * w], off);
      issue_rows16(dlt, &S.ndelta[16 * w], off);
    }
  };
  auto compute = [&](auto st, int) {
    const LocStage32<DP>& S = stage(st);
    // dp = <dO, V> - delta: the products accumulate onto -delta; slots 4j .. 4j+3 are
    // rows 32qh + 8j + 4half + e
    f32x16 s, dp, nd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 d4 = *(const f32x4*)&S.ndelta[32 * qh + 8 * j + 4 * half];
#pragma unroll
      for (int e = 0; e < 4; ++e) nd[4 * j + e] = d4[e];
    }
    score32_pair(S.q, kf, s, S.g, vf, dp, col, half, qh, nd);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *(const f32x4*)&S.lse2[32 * qh + 8 * j + 4 * half];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[4 * j + e], c, -l4[e]));
        s[4 * j + e] = p;
        dp[4 * j + e] = p * dp[4 * j + e];
      }
    }
    accum32_rows(S.g, s, dv, lane, half, qh);
    accum32_rows(S.q, dp, dk, lane, half, qh);
  };
  pipeline_lds<kLdsStages, 2 * Dma::ROUNDS + 2>(ntiles, issue, compute);
  __syncthreads();  // the partial and staging buffers overlay the stages

  constexpr int NDT = DP / 32;
  if constexpr (DP == 96) {
    if (a.D == 96) {
      local32_epilogue96(a, dk, dv, (f32x4*)(kh == 0 ? (void*)&s0 : (void*)&s1), b, h, kb, krow0, kloc, nk,
                         qh, lane, half);
      return;
    }
  }
  f32x4* part = (f32x4*)(kh == 0 ? (void*)&s0 : (void*)&s1);  // [slot][lane]
  float(*st)[DP + 1] = (float(*)[DP + 1]) & s2;
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        part[(4 * dt + q) * 64 + lane] = f32x4{dk[dt][4 * q], dk[dt][4 * q + 1], dk[dt][4 * q + 2], dk[dt][4 * q + 3]};
        part[(4 * NDT + 4 * dt + q) * 64 + lane] =
            f32x4{dv[dt][4 * q], dv[dt][4 * q + 1], dv[dt][4 * q + 2], dv[dt][4 * q + 3]};
      }
    }
  }
  __syncthreads();
  // epilogue (query half 0 holds the totals): dK~ = scale * acc + dKbar / |b| (then R^T),
  // dV = acc + dVbar / |b|, each staged through LDS rows and scattered to packed order
  const float inv = block_inv(a, b, kb);
  const float* dkb = a.dkbar + (bh * a.nblkp + kb) * DP;
  const float* dvb = a.dvbar + (bh * a.nblkp + kb) * DP;
  if (qh == 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 pk = part[(4 * dt + q) * 64 + lane];
        const f32x4 pv = part[(4 * NDT + 4 * dt + q) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[dt][4 * q + e] += pk[e];
          dv[dt][4 * q + e] += pv[e];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * dt + 8 * (i >> 2) + 4 * half + (i & 3);
        st[kloc][d] = dk[dt][i] * a.scale + (a.with_summaries ? dkb[d] * inv : 0.f);
      }
    }
  }
  __syncthreads();
  write_rows<bf16>(a, &st[0][0], DP + 1, nk, b, h, krow0, true, (bf16*)a.dk, sm.src, sm.rel);
  if (qh == 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * dt + 8 * (i >> 2) + 4 * half + (i & 3);
        st[kloc][d] = dv[dt][i] + (a.with_summaries ? dvb[d] * inv : 0.f);
      }
    }
  }
  __syncthreads();
  write_rows<bf16>(a, &st[0][0], DP + 1, nk, b, h, krow0, false, (bf16*)a.dv, sm.src, sm.rel);
}

// ---------------------------------------------------------------------------------
// bwd_summary for bf16 with 32 summary columns per wave (Dp 32, 96), fed by direct LDS
// copies as bwd_local32 is: workgroup = (64 summaries, head, volume x query chunk), four
// waves = summary half kh x query-row half qh of every query tile.  A summary's
// probability is zero for the query blocks it is local to (and for the padding
// summaries past the last block).  The two query halves' partial dKbar~, dVbar are added
// through LDS and written as the chunk's partial rows, as bwd_summary does.
// ---------------------------------------------------------------------------------
template <int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_summary32(BwdArgs a) {
  // one LDS object per stage; the epilogue reuses stages 0 / 1 for query half 1's partial
  // sums of summary half 0 / 1 ([slot][lane] float4s)
  __shared__ LocStage32<DP> s0, s1, s2;
  static_assert(sizeof(f32x4) * DP / 32 * 8 * 64 <= sizeof(LocStage32<DP>), "partials fit a stage");
  // 1-D grid over (summary tile, chunk, head, volume), summary tile fastest
  const int nst = a.nblkp / kTile;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int r0 = (L % nst) * kTile, chunk = (L / nst) % a.chunks;
  const int h = (L / nst / a.chunks) % a.H, b = L / nst / a.chunks / a.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int sid = r0 + 32 * kh + col;  // this lane's summary (block id); padding rows are zero
  ColFrag32<DP> kf, vf;
  kf.load((const bf16*)a.kbar + (bh * a.nblkp + sid) * DP, true, half);
  vf.load((const bf16*)a.vbar + (bh * a.nblkp + sid) * DP, true, half);
  const int32_t* g = a.geom + b * G_FIELDS;
  // the volume's block grid covers its bounding box: ceil(extent / b) blocks per axis
  const int nby = (g[G_EY] + a.by - 1) / a.by, nbx = (g[G_EX] + a.bx - 1) / a.bx;
  const int sz = sid / (nby * nbx), sy = (sid / nbx) % nby, sx = sid % nbx;
  f32x16 dk[DP / 32], dv[DP / 32];
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) dk[dt] = dv[dt] = f32x16{};

  const int q_begin = (int)((int64_t)chunk * a.nblk / a.chunks);
  const int q_end = (int)((int64_t)(chunk + 1) * a.nblk / a.chunks);
  const int nrow = bvol < kTile ? bvol : kTile;
  const int tpb = a.tiles_per_block;
  const size_t slice = (size_t)N * DP * sizeof(bf16);
  const Src qrot((const bf16*)a.qrot + bh * N * DP, slice);
  const Src doc((const bf16*)a.doc + bh * N * DP, slice);
  const Src lsec(a.lsec + bh * N, (size_t)N * sizeof(float));
  const Src dlt(a.ndelta + bh * N, (size_t)N * sizeof(float));
  const float c = a.scale_log2;
  // tile t = (query block q_begin + t / tpb, sub-tile t % tpb); rows past a block of fewer
  // than 64 tokens arrive as zeros (Q = dO = 0 there, so they add nothing)
  const int ntiles = (q_end - q_begin) * tpb;
  using Dma = TileDma<DP, kThreads>;
  const Dma dma;
  auto stage = [&](auto st) -> LocStage32<DP>& {
    if constexpr (decltype(st)::value == 0) return s0;
    else if constexpr (decltype(st)::value == 1) return s1;
    else return s2;
  };
  // Tiles are issued, and computed, in increasing order, so cursors replace the divisions
  // (scalar code, but issued by this wave) that would find each tile's query block and
  // its block-grid coordinates.
  int iss_q = q_begin, iss_s = 0;  // next tile to issue: query block, sub-tile
  int cmp_s = 0;                   // sub-tile of the next tile to compute
  int qz = q_begin / (nby * nbx), qy = (q_begin / nbx) % nby, qx = q_begin % nbx;  // its block
  auto issue = [&](auto st, int t) {
    LocStage32<DP>& S = stage(st);
    const int row0 = iss_q * bvol + iss_s * kTile;
    if (++iss_s == tpb) {
      iss_s = 0;
      ++iss_q;
    }
    const int w = wave_id(), r = 16 * w + (lane & 15);
    if (nrow == kTile) {
      dma.issue_at(qrot, S.q, (uint32_t)row0 * DP);
      dma.issue_at(doc, S.g, (uint32_t)row0 * DP);
    } else {
      dma.issue(qrot, S.q, nrow, [&](int rr) { return (row0 + rr) * DP; });
      dma.issue(doc, S.g, nrow, [&](int rr) { return (row0 + rr) * DP; });
    }
    const uint32_t off = r < nrow ? (uint32_t)(row0 + r) * 4u : 0x80000000u;
    issue_rows16(lsec, &S.lse2[16 * w], off);
    issue_rows16(dlt, &S.ndelta[16 * w], off);
  };
  auto compute = [&](auto st, int t) {
    const LocStage32<DP>& S = stage(st);
    const int cheb = max(max(abs(qz - sz), abs(qy - sy)), abs(qx - sx));
    const bool masked = sid >= a.nblk || cheb <= a.radius;  // per lane: this summary column
    if (++cmp_s == tpb) {  // the next tile starts the next query block (raster order)
      cmp_s = 0;
      if (++qx == nbx) {
        qx = 0;
        if (++qy == nby) {
          qy = 0;
          ++qz;
        }
      }
    }
    // dp = <dO, Vbar> - delta: the products accumulate onto -delta; slots 4j .. 4j+3 are
    // rows 32qh + 8j + 4half + e
    f32x16 s, dp, nd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 d4 = *(const f32x4*)&S.ndelta[32 * qh + 8 * j + 4 * half];
#pragma unroll
      for (int e = 0; e < 4; ++e) nd[4 * j + e] = d4[e];
    }
    score32_pair(S.q, kf, s, S.g, vf, dp, col, half, qh, nd);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *(const f32x4*)&S.lse2[32 * qh + 8 * j + 4 * half];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = fast_exp2(fmaf(s[4 * j + e], c, -l4[e]));
        if (masked) p = 0.f;
        s[4 * j + e] = p;
        dp[4 * j + e] = p * dp[4 * j + e];
      }
    }
    accum32_rows(S.g, s, dv, lane, half, qh);
    accum32_rows(S.q, dp, dk, lane, half, qh);
  };
  pipeline_lds<kLdsStages, 2 * Dma::ROUNDS + 2>(ntiles, issue, compute);
  __syncthreads();  // the partial sums below overlay the stages

  constexpr int NDT = DP / 32;
  f32x4* part = (f32x4*)(kh == 0 ? (void*)&s0 : (void*)&s1);
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        part[(4 * dt + q) * 64 + lane] = f32x4{dk[dt][4 * q], dk[dt][4 * q + 1], dk[dt][4 * q + 2], dk[dt][4 * q + 3]};
        part[(4 * NDT + 4 * dt + q) * 64 + lane] =
            f32x4{dv[dt][4 * q], dv[dt][4 * q + 1], dv[dt][4 * q + 2], dv[dt][4 * q + 3]};
      }
  }
  __syncthreads();
  if (qh == 1) return;
  // value of dim 32dt + 8jj + 4half + e is slot 4jj + e of block dt
  const int64_t base = (((int64_t)chunk * a.B * a.H + bh) * a.nblkp + sid) * DP;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 pk = part[(4 * dt + jj) * 64 + lane], pv = part[(4 * NDT + 4 * dt + jj) * 64 + lane];
      f32x4 ok, ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[e] = (dk[dt][4 * jj + e] + pk[e]) * a.scale;
        ov[e] = dv[dt][4 * jj + e] + pv[e];
      }
      *(f32x4*)(a.part_k + base + 32 * dt + 8 * jj + 4 * half) = ok;
      *(f32x4*)(a.part_v + base + 32 * dt + 8 * jj + 4 * half) = ov;
    }
}

// ---------------------------------------------------------------------------------
// bwd_dq: workgroup = (64 queries of one block, head, volume)
// ---------------------------------------------------------------------------------
// Local key tiles whose live-row masks bwd_dq precomputes when slots can be empty.
constexpr int kDqLiveTiles = 512;

template <typename T, int DP>
struct DqSmem {
  union {
    struct {
      RowTile<T, DP> k, v;
    } t;
    float st[kTile][DP + 1];
  } u;
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  uint64_t live[kDqLiveTiles];  // local tile t: bit r = key row r holds a token (empty slots only)
  int nloc;
  int src[kTile], rel[kTile * 3];
};

// Bit r of `live` says whether tile row r is a real, unmasked key.
template <typename T, int DP>
__device__ inline void dq_step(const DqSmem<T, DP>& sm, const ColFrag<T, DP>& qf, const ColFrag<T, DP>& gf,
                               f32x4 (&dq)[DP / 16], float lse2, float ndelta, float c, int col, int grp,
                               uint64_t live) {
  f32x4 s[4], dp[4];
  score(sm.u.t.k, qf, s, col, grp);
  // dp = <dO, V> - delta: the products accumulate onto -delta (one value per lane's query)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) dp[mt] = f32x4{ndelta, ndelta, ndelta, ndelta};
  score_acc(sm.u.t.v, gf, dp, col, grp);
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
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(fmaf(s[mt][i], c, -lse2));
      dp[mt][i] = p * dp[mt][i];
    }
  }
  accum(sm.u.t.k, dp, dq, col, grp);
}

// Epilogue of bwd_dq for D = 96, in registers: lane (query, group g) holds dims
// 16dt + 4g + i, so the rotation pair (k, k + 16) of axis ax is blocks 2ax and 2ax + 1 of
// the same lane; dq = R^T (scale * acc) is stored as 4-element pieces.
template <typename T>
__device__ inline void dq_epilogue96(const BwdArgs& a, f32x4 (&dq)[6], int b, int h, int row, bool ok, int grp) {
  if (!ok) return;
  const int src = a.perm[(int64_t)b * a.NC + row];
  if (src < 0) return;  // empty slot
  const int64_t tok0 = a.voff[b];
  const int32_t* g = a.geom + b * G_FIELDS;
  const int32_t* c = a.coords + (tok0 + src) * 3;
  T* dst = (T*)a.dq + (tok0 + src) * a.grad_stride + (int64_t)h * 96;
  if (a.pos_mode == PACK3D_POS_PACKED_1D) {  // pairs (k, k + 48): dq[dt] with dq[dt + 3]
    const float2* cs = a.tab + (int64_t)src * 48 + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      Vec<T, 4> lo4, hi4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 t = cs[16 * dt + i];
        const float lo = dq[dt][i] * a.scale, hi = dq[dt + 3][i] * a.scale;
        lo4.v[i] = (T)(lo * t.x + hi * t.y);
        hi4.v[i] = (T)(-lo * t.y + hi * t.x);
      }
      *(Vec<T, 4>*)(dst + 16 * dt + 4 * grp) = lo4;
      *(Vec<T, 4>*)(dst + 48 + 16 * dt + 4 * grp) = hi4;
    }
    return;
  }
  if (a.pos_mode == PACK3D_POS_NONE) {
#pragma unroll
    for (int dt = 0; dt < 6; ++dt) {
      Vec<T, 4> v4;
#pragma unroll
      for (int i = 0; i < 4; ++i) v4.v[i] = (T)(dq[dt][i] * a.scale);
      *(Vec<T, 4>*)(dst + 16 * dt + 4 * grp) = v4;
    }
    return;
  }
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) {
    int r = c[ax] - g[G_OZ + ax];
    r = r < 0 ? 0 : (r >= a.trows ? a.trows - 1 : r);
    const float2* cs = a.tab + (int64_t)r * 16 + 4 * grp;  // 16 pairs per axis
    Vec<T, 4> lo4, hi4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 t = cs[i];
      const float lo = dq[2 * ax][i] * a.scale, hi = dq[2 * ax + 1][i] * a.scale;
      lo4.v[i] = (T)(lo * t.x + hi * t.y);   // y1 c + y2 s
      hi4.v[i] = (T)(-lo * t.y + hi * t.x);  // -y1 s + y2 c
    }
    *(Vec<T, 4>*)(dst + 32 * ax + 4 * grp) = lo4;
    *(Vec<T, 4>*)(dst + 32 * ax + 16 + 4 * grp) = hi4;
  }
}

// three waves per SIMD where the registers allow it (a wider head dim would spill)
template <typename T, int DP, bool ONE_BLOCK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DP * sizeof(T) <= 192 ? 3 : 2)))
void k_bwd_dq(BwdArgs a) {
  __shared__ DqSmem<T, DP> sm;
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int qb = tile / a.tiles_per_block, qs = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nq = bvol < kTile ? bvol : kTile;
  const int qrow0 = qb * bvol + qs * kTile;
  const int qloc = 16 * wave + col;
  const bool qok = qloc < nq;
  const uint32_t* occ = a.occ + (int64_t)b * a.occ_words;
  if (a.holes && !any_occupied(occ, qrow0, nq)) return;  // no token among the tile's queries
  ColFrag<T, DP> qf, gf;
  qf.load((const T*)a.qrot + (bh * N + qrow0 + qloc) * DP, qok, grp);
  gf.load((const T*)a.doc + (bh * N + qrow0 + qloc) * DP, qok, grp);
  const float lse2 = qok ? a.lsec[bh * N + qrow0 + qloc] : INFINITY;
  const float ndelta = qok ? a.ndelta[bh * N + qrow0 + qloc] : 0.f;

  const int mask_words = a.nblkp / 32;
  // summaries: empty blocks start masked (as in the forward), the local blocks are added below
  for (int i = tid; i < mask_words; i += kThreads) sm.mask[i] = a.holes ? a.emask[(int64_t)b * mask_words + i] : 0u;
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + qb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = sm.nloc;
  for (int i = tid; i < nloc; i += kThreads) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));
  f32x4 dq[DP / 16];
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t slice = (size_t)N * DP * sizeof(T), sslice = (size_t)a.nblkp * DP * sizeof(T);
  const Src krot((const T*)a.krot + bh * N * DP, slice);
  const Src vrow((const T*)a.vr + bh * N * DP, slice);
  const Src kbar((const T*)a.kbar + bh * a.nblkp * DP, sslice);
  const Src vbar((const T*)a.vbar + bh * a.nblkp * DP, sslice);
  const float c = a.scale_log2;
  const int nkeys = nloc * bvol;
  const int nlt = (nkeys + kTile - 1) / kTile;
  const int total = nlt + (a.with_summaries ? a.nblkp / kTile : 0);
  // With empty slots the local tiles' live-row masks come from the occupancy bits.  They are
  // taken here, one tile per wave at a time, because a load of occupancy words inside the
  // pipeline would also wait for the tile loads in flight.
  const bool live_table = a.holes && nlt <= kDqLiveTiles;
  if (live_table) {
    for (int t = wave; t < nlt; t += kThreads / 64) {
      const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
      const uint64_t lv = occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
      if (lane == 0) sm.live[t] = lv;
    }
    __syncthreads();
  }
  struct Stage {
    RowRegs<T, DP> k, v;
  } st0, st1;
  // ONE_BLOCK: local tiles are fetched in order, so a cursor (entry of the neighbour list,
  // 64-row tile within that block) replaces a division per tile
  const int tpb = a.tiles_per_block;
  int cur_entry = 0, cur_sub = 0;
  auto fetch = [&](Stage& S, int t) {
    if (t < nlt) {
      const int j0 = t * kTile;
      const int valid = nkeys - j0 < kTile ? nkeys - j0 : kTile;
      if constexpr (ONE_BLOCK) {
        const int row0 = __builtin_amdgcn_readfirstlane(sm.list[cur_entry]) * bvol + cur_sub * kTile;
        if (++cur_sub == tpb) {
          cur_sub = 0;
          ++cur_entry;
        }
        S.k.fetch_at(krot, (uint32_t)row0 * DP);
        S.v.fetch_at(vrow, (uint32_t)row0 * DP);
      } else {
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
    S.k.store(sm.u.t.k);
    S.v.store(sm.u.t.v);
  };
  auto compute = [&](int t) {
    uint64_t live;
    if (t < nlt) {
      const int valid = nkeys - t * kTile < kTile ? nkeys - t * kTile : kTile;
      live = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
      if (live_table) live &= sm.live[t];
      else if (a.holes) live &= occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), valid);
    } else {
      const int ts = t - nlt, r0 = ts * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * ts + 1] << 32) | sm.mask[2 * ts];
      live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
    }
    if (live == 0ull) return;
    dq_step(sm, qf, gf, dq, lse2, ndelta, c, col, grp, live);
  };
  pipeline2(total, st0, st1, fetch, store, compute);
  if constexpr (DP == 96) {
    if (a.D == 96) {
      dq_epilogue96<T>(a, dq, b, h, qrow0 + qloc, qok, grp);
      return;
    }
  }
  __syncthreads();  // the staging area below overlays the tiles
#pragma unroll
  for (int dt = 0; dt < DP / 16; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.u.st[qloc][16 * dt + 4 * grp + i] = dq[dt][i] * a.scale;
  }
  __syncthreads();
  write_rows<T>(a, &sm.u.st[0][0], DP + 1, nq, b, h, qrow0, true, (T*)a.dq, sm.src, sm.rel);
}

// ---------------------------------------------------------------------------------
// bwd_dq for bf16 at D = 96 with blocks of 64-token multiples: 32 query columns per wave,
// fed by direct LDS copies.  Workgroup = (64 queries, head, volume), four waves: query half
// qh = wave >> 1 (the wave's 32 queries are the B operand, in registers) and key half
// kh = wave & 1 of every key tile.  Per tile a wave forms S^T = K Q^T and dP^T = V dO^T - delta
// for its 32 keys (v_mfma_f32_32x32x16_bf16), dS = P * dP, and dQ^T += K^T dS^T with K read
// transposed.  The 32x32 products read half the LDS bytes per multiply of the 16-column
// kernel, which is bound by LDS bandwidth.  K and V tiles arrive by direct copies into two
// stages (separate LDS objects, so plain reads of one stage do not wait for copies into the
// other); the transposed K operands are read by one asm block that waits only for its own
// reads.  The two key halves' partial dQ are added through LDS before the epilogue.
// ---------------------------------------------------------------------------------
constexpr int kDq32LiveTiles = 32;

struct DqSmem32 {
  int list[kMaxSlots];
  uint32_t mask[kMaxBlocks / 32];
  uint64_t live[kDq32LiveTiles];  // local tile t: bit r = key row r holds a token (empty slots only)
  int nloc;
};

template <int DP>
struct DqStage32 {
  RowTile<bf16, DP> k, v;
};

// Epilogue for D = 96: lane (query col, half h) holds dims 32dt + 8(i/4) + 4h + i%4 in slot i
// of block dt, so each rotation pair (k, k + 16 of an axis group; k, k + 48 in 1D) sits in one
// lane; dq = R^T (scale * acc) is stored as 8-byte pieces.
__device__ inline void dq32_epilogue96(const BwdArgs& a, f32x16 (&acc)[3], int b, int h, int row, bool ok,
                                       int half) {
  if (!ok) return;
  const int src = a.perm[(int64_t)b * a.NC + row];
  if (src < 0) return;  // empty slot
  const int64_t tok0 = a.voff[b];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] *= a.scale;
  if (a.pos_mode == PACK3D_POS_AXIAL) {
    const int32_t* g = a.geom + b * G_FIELDS;
    const int32_t* c = a.coords + (tok0 + src) * 3;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      int r = c[dt] - g[G_OZ + dt];
      r = r < 0 ? 0 : (r >= a.trows ? a.trows - 1 : r);
      const float2* cs = a.tab + (int64_t)r * 16 + 4 * half;  // 16 pairs per axis
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 t = cs[8 * j + e];
          const float lo = acc[dt][4 * j + e], hi = acc[dt][4 * j + 8 + e];
          acc[dt][4 * j + e] = lo * t.x + hi * t.y;       // y1 c + y2 s
          acc[dt][4 * j + 8 + e] = -lo * t.y + hi * t.x;  // -y1 s + y2 c
        }
    }
  } else if (a.pos_mode == PACK3D_POS_PACKED_1D) {
    const float2* cs = a.tab + (int64_t)src * 48 + 4 * half;  // 48 pairs (k, k + 48) per row
#pragma unroll
    for (int m = 0; m < 6; ++m)  // dims 8m + 4 half + e and 8(m + 6) + 4 half + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 t = cs[8 * m + e];
        const float y1 = acc[m / 4][4 * (m % 4) + e], y2 = acc[(m + 6) / 4][4 * ((m + 6) % 4) + e];
        acc[m / 4][4 * (m % 4) + e] = y1 * t.x + y2 * t.y;
        acc[(m + 6) / 4][4 * ((m + 6) % 4) + e] = -y1 * t.y + y2 * t.x;
      }
  }
  bf16* dst = (bf16*)a.dq + (tok0 + src) * a.grad_stride + (int64_t)h * 96;
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      *(bf16x4*)(dst + 32 * dt + 8 * jj + 4 * half) =
          bf16x4{(bf16)acc[dt][4 * jj], (bf16)acc[dt][4 * jj + 1], (bf16)acc[dt][4 * jj + 2], (bf16)acc[dt][4 * jj + 3]};
}

template <int DP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void k_bwd_dq32(BwdArgs a) {
  static_assert(DP == 96, "the transposed reads and the epilogue are written for D = 96");
  __shared__ DqSmem32 sm;
  __shared__ DqStage32<DP> s0, s1;
  static_assert(sizeof(f32x4) * (4 * DP / 32) * 64 * 2 <= sizeof(DqStage32<DP>), "partial dq fits a stage");
  const int ntile = a.nblk * a.tiles_per_block;
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int tile = L % ntile, h = (L / ntile) % a.H, b = L / ntile / a.H;
  const int qb = tile / a.tiles_per_block, qs = tile - qb * a.tiles_per_block;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  const int N = a.NC, bvol = a.bvol;
  const int64_t bh = (int64_t)b * a.H + h;
  const int qrow0 = qb * bvol + qs * kTile;  // bvol is a multiple of 64: 64 queries per tile
  const int qloc = 32 * qh + col;
  const uint32_t* occ = a.occ + (int64_t)b * a.occ_words;
  if (a.holes && !any_occupied(occ, qrow0, kTile)) return;  // no token among the tile's queries
  ColFrag32<DP> qf, gf;
  qf.load((const bf16*)a.qrot + (bh * N + qrow0 + qloc) * DP, true, half);
  gf.load((const bf16*)a.doc + (bh * N + qrow0 + qloc) * DP, true, half);
  const float lse2 = a.lsec[bh * N + qrow0 + qloc];   // +inf at an empty slot: P = 0
  const float ndelta = a.ndelta[bh * N + qrow0 + qloc];

  const int mask_words = a.nblkp / 32;
  for (int i = tid; i < mask_words; i += kThreads) sm.mask[i] = a.holes ? a.emask[(int64_t)b * mask_words + i] : 0u;
  if (wave == 0) compact_neighbours(a.nbr + ((int64_t)b * a.nblk + qb) * a.slots, a.slots, sm.list, &sm.nloc);
  __syncthreads();
  const int nloc = __builtin_amdgcn_readfirstlane(sm.nloc);
  for (int i = tid; i < nloc; i += kThreads) atomicOr(&sm.mask[sm.list[i] >> 5], 1u << (sm.list[i] & 31));
  const int nkeys = nloc * bvol;
  const int nlt = nkeys / kTile;
  const int total = nlt + (a.with_summaries ? a.nblkp / kTile : 0);
  // with empty slots the local tiles' occupancy is read before any copy is in flight
  const bool live_table = a.holes && nlt <= kDq32LiveTiles;
  if (live_table) {
    for (int t = wave; t < nlt; t += kThreads / 64) {
      const uint64_t lv = occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), kTile);
      if (lane == 0) sm.live[t] = lv;
    }
  }
  wait_vm<0>();  // the query rows, lse and delta are in registers before any copy starts
  f32x16 dq[DP / 32];
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) dq[dt] = f32x16{};
  const float c = a.scale_log2;

  const size_t es = sizeof(bf16);
  const bf16* kq = (const bf16*)a.krot + bh * N * DP;
  const bf16* vq = (const bf16*)a.vr + bh * N * DP;
  const bf16* kbq = (const bf16*)a.kbar + bh * a.nblkp * DP;
  const bf16* vbq = (const bf16*)a.vbar + bh * a.nblkp * DP;
  const size_t bytes_loc = (size_t)N * DP * es, bytes_sum = (size_t)a.nblkp * DP * es;
  using Dma = TileDma<DP, kThreads>;
  const Dma dma;
  auto stage = [&](auto sg) -> DqStage32<DP>& {
    if constexpr (decltype(sg)::value == 0) return s0;
    else return s1;
  };
  // tiles are issued in order, so a cursor (entry of the neighbour list, 64-row tile within
  // that block) replaces a division per tile
  const int tpb = a.tiles_per_block;
  int cur_entry = 0, cur_sub = 0;
  auto issue = [&](DqStage32<DP>& S, int t) {
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
  };
  // this wave's live key rows of tile t (bit r: row 32kh + r)
  auto live_rows = [&](int t) -> uint32_t {
    uint64_t live;
    if (t < nlt) {
      live = a.holes ? (live_table ? sm.live[t] : occupied_rows(occ, VirtualRows(sm.list, bvol, t * kTile), kTile))
                     : ~0ull;
    } else {
      const int ts = t - nlt, r0 = ts * kTile;
      const int rows = a.nblk - r0 < kTile ? a.nblk - r0 : kTile;
      const uint64_t used = ((uint64_t)sm.mask[2 * ts + 1] << 32) | sm.mask[2 * ts];
      live = (rows >= 64 ? ~0ull : ((1ull << rows) - 1ull)) & ~used;
    }
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(kh ? (uint32_t)(live >> 32) : (uint32_t)live));
  };
  auto compute = [&](auto sg, uint32_t mine) {
    const DqStage32<DP>& S = stage(sg);
    // S^T and dP^T for keys 32kh .. 32kh+31; dS = P (dP - delta), with -delta added here (a
    // register block of it as the accumulators' start would stay live across the loop)
    f32x16 s, dp;
    score32_pair_ahead<DP, 3>(S.k, qf, s, S.v, gf, dp, col, half, kh);
    if (mine != ~0u) mask_rows32(s, mine, half);
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p0 = fast_exp2(fmaf(s[2 * j], c, -lse2)), p1 = fast_exp2(fmaf(s[2 * j + 1], c, -lse2));
      pb[j >> 2][2 * (j & 3)] = (bf16)(p0 * (dp[2 * j] + ndelta));
      pb[j >> 2][2 * (j & 3) + 1] = (bf16)(p1 * (dp[2 * j + 1] + ndelta));
    }
    RowsFrag32<DP> kfr;
    read_rows32_96(S.k, kfr, lane, half, kh);  // this stage landed; copies in flight target the other
    accum32_packed(kfr, pb, dq);
  };
  auto step = [&](auto sg, int t) {
    constexpr int SI = decltype(sg)::value;
    wait_vm<0>();
    barrier_copies();  // tile t is in stage SI; every wave is done with the other stage
    const uint32_t mine = live_rows(t);
    if (t + 1 < total) issue(stage(Stage_<1 - SI>{}), t + 1);
    if (mine) compute(sg, mine);
  };
  if (total > 0) issue(s0, 0);
  for (int t = 0; t < total; t += 2) {
    step(Stage_<0>{}, t);
    if (t + 1 < total) step(Stage_<1>{}, t + 1);
  }
  __syncthreads();  // stage 0 is reused for the key halves' partial dq
  f32x4* part = (f32x4*)&s0 + qh * (4 * DP / 32) * 64;  // [qh][slot][lane]
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[(4 * dt + q) * 64 + lane] = f32x4{dq[dt][4 * q], dq[dt][4 * q + 1], dq[dt][4 * q + 2], dq[dt][4 * q + 3]};
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 o = part[(4 * dt + q) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) dq[dt][4 * q + e] += o[e];
    }
  dq32_epilogue96(a, dq, b, h, qrow0 + qloc, true, half);
}

// Explicit instantiations of the 32-column kernels: when several kernels of this file call
// the copy helpers from generic lambdas, the host compilation can leave out the launch stub
// of some of them with no diagnostic (the library then fails to load); instantiating every
// one here makes the host side emit all of them.
template __global__ void k_bwd_local32<32, true>(BwdArgs);
template __global__ void k_bwd_local32<96, true>(BwdArgs);
template __global__ void k_bwd_local32<32, false>(BwdArgs);
template __global__ void k_bwd_local32<96, false>(BwdArgs);
template __global__ void k_bwd_summary32<32, true>(BwdArgs);
template __global__ void k_bwd_summary32<96, true>(BwdArgs);
template __global__ void k_bwd_summary32<32, false>(BwdArgs);
template __global__ void k_bwd_summary32<96, false>(BwdArgs);
template __global__ void k_bwd_dq32<96>(BwdArgs);

template <typename T, int DP, bool ONE_BLOCK>
pack3d_status launch_dp(const Dims& d, const BwdArgs& a, hipStream_t s) {
  const dim3 tiles(d.nblk * a.tiles_per_block * d.H * d.B);
  if (a.with_summaries) {
    {
      ProfileScope prof("bwd_summary", s);
      const dim3 grid(d.nblkp / kTile * a.chunks * d.H * d.B);
      // 32-column waves with direct LDS copies for bf16 where rows need no padding
      if constexpr (sizeof(T) == 2 && (DP == 32 || DP == 96))
        hipLaunchKernelGGL((k_bwd_summary32<DP, ONE_BLOCK>), grid, dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((k_bwd_summary<T, DP, ONE_BLOCK>), grid, dim3(kThreads), 0, s, a);
    }
    const int64_t n = (int64_t)d.B * d.H * d.nblkp * d.Dp;
    ProfileScope prof("bwd_reduce", s);
    hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)a.part_k, (const float*)a.part_v, a.dkbar, a.dvbar, n, a.chunks);
  }
  {
    ProfileScope prof("bwd_local", s);
    // 32-column waves with direct LDS copies for bf16 where rows need no padding
    if constexpr (sizeof(T) == 2 && (DP == 32 || DP == 96))
      hipLaunchKernelGGL((k_bwd_local32<DP, ONE_BLOCK>), tiles, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_bwd_local<T, DP, ONE_BLOCK>), tiles, dim3(kThreads), 0, s, a);
  }
  {
    ProfileScope prof("bwd_dq", s);
    // 32-column waves with direct copies for bf16 at D = 96 in blocks of 64-token multiples.
    // Position mode "none" keeps the register-staged kernel: earlier direct-copy versions of
    // this kernel raised memory faults in that mode only, with the cause not found.
    if constexpr (sizeof(T) == 2 && DP == 96 && ONE_BLOCK) {
      if (d.D == 96 && a.pos_mode != PACK3D_POS_NONE) hipLaunchKernelGGL(k_bwd_dq32<96>, tiles, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((k_bwd_dq<T, DP, ONE_BLOCK>), tiles, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_bwd_dq<T, DP, ONE_BLOCK>), tiles, dim3(kThreads), 0, s, a);
    }
  }
  return check_launch("backward: attention");
}

template <typename T, int DP>
pack3d_status launch_dp(const Dims& d, const BwdArgs& a, hipStream_t s) {
  return d.bvol % kTile == 0 ? launch_dp<T, DP, true>(d, a, s) : launch_dp<T, DP, false>(d, a, s);
}

template <typename T>
pack3d_status launch_typed(const Dims& d, const BwdArgs& a, hipStream_t s) {
  // all heads per workgroup where bf16 rows need no padding and a slot's pieces fit the items
  const int per_slot = d.H * (d.D / 8);
  const int tpw = sizeof(T) == 2 && d.Dp == d.D && d.half % 8 == 0 ? 256 * kPreItems / per_slot : 0;
  if (tpw > 0) {
    const dim3 grid((unsigned)((d.NC + tpw - 1) / tpw), d.B);
    ProfileScope prof("bwd_pre", s);
    hipLaunchKernelGGL(k_bwd_pre_rows, grid, dim3(256), sizeof(float) * 256 * kPreItems, s, a, tpw);
  } else {
    const int ntok = d.bvol < kTile ? d.bvol : kTile;
    int vec = 1;
    const int cap = 16 / (int)sizeof(T);
    while (vec * 2 <= cap && d.half % (vec * 2) == 0) vec *= 2;
    const size_t lds = sizeof(float) * ntok * (d.D / vec);
    const dim3 grid(d.nblk, d.H, d.B);
    ProfileScope prof("bwd_pre", s);
    switch (vec) {
      case 1: hipLaunchKernelGGL((k_bwd_pre<T, 1>), grid, dim3(256), lds, s, a); break;
      case 2: hipLaunchKernelGGL((k_bwd_pre<T, 2>), grid, dim3(256), lds, s, a); break;
      case 4: hipLaunchKernelGGL((k_bwd_pre<T, 4>), grid, dim3(256), lds, s, a); break;
      default:
        if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((k_bwd_pre<T, 8>), grid, dim3(256), lds, s, a);
        break;
    }
  }
  pack3d_status st = check_launch("backward: preprocess");
  if (st != PACK3D_OK) return st;
  switch (d.Dp) {
    case 32: return launch_dp<T, 32>(d, a, s);
    case 64: return launch_dp<T, 64>(d, a, s);
    case 96: return launch_dp<T, 96>(d, a, s);
    case 128: return launch_dp<T, 128>(d, a, s);
    default: return set_error(PACK3D_E_UNSUPPORTED, "backward: padded head dim %d", d.Dp);
  }
}

}  // namespace

pack3d_status launch_attn_bwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at, const int32_t* coords,
                              const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              char* ws, const Workspace& w, hipStream_t s) {
  BwdArgs a;
  a.qrot = ws + w.qrot; a.krot = ws + w.krot; a.vr = ws + w.vr; a.kbar = ws + w.kbar; a.vbar = ws + w.vbar;
  a.doc = ws + w.doc; a.lsec = (float*)(ws + w.lsec); a.ndelta = (float*)(ws + w.delta);
  a.dkbar = (float*)(ws + w.dkbar); a.dvbar = (float*)(ws + w.dvbar);
  a.part_k = (float*)(ws + w.part_k); a.part_v = (float*)(ws + w.part_v);
  a.tab = (const float2*)(ws + w.rope);
  a.out = out; a.lse = lse; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.coords = coords; a.perm = ix->perm; a.nbr = ix->nbr; a.geom = ix->geom;
  a.voff = ix->voff; a.count = ix->count; a.occ = ix->occ; a.emask = ix->emask;
  a.holes = d.holes; a.occ_words = ix->occ_words;
  a.grad_stride = d.grad_stride;
  a.B = d.B; a.NC = d.NC; a.Nmax = d.Nmax; a.H = d.H; a.D = d.D; a.Dp = d.Dp; a.nblk = d.nblk; a.nblkp = d.nblkp; a.bvol = d.bvol;
  a.slots = d.slots; a.radius = ix->radius;
  a.tiles_per_block = d.bvol > kTile ? d.bvol / kTile : 1;
  a.with_summaries = at->with_summaries ? 1 : 0;
  a.chunks = summary_chunks(d);
  a.pos_mode = d.pos_mode; a.groups = d.groups; a.gw = d.gw; a.half = d.half; a.trows = d.trows;
  a.bz = ix->block[0]; a.by = ix->block[1]; a.bx = ix->block[2];
  a.scale = at->softmax_scale > 0.f ? at->softmax_scale : 1.0f / std::sqrt((float)d.D);
  a.scale_log2 = a.scale * kLog2e;
  return at->dtype == PACK3D_BF16 ? launch_typed<bf16>(d, a, s) : launch_typed<float>(d, a, s);
}

}  // namespace pack3d
