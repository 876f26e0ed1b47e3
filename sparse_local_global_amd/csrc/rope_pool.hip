// K1 + K2: axial RoPE, gather into canonical order, and block mean pooling.
//
// "Geometry Matters in Packed 3D Attention" (abstract): every query-key and
// query-summary interaction is indexed by axial RoPE on the true token-grid
// coordinates, and the rotation is applied before a block is summarized.  So for
// each token the head dim is cut into three contiguous groups (z, y, x) of width
// d_a = D/3, element k of a group pairs with element k + d_a/2 and both turn by
// angle coord_a * theta_k with theta_k = base^(-2k/d_a) (the frequency set and
// half-split pairing of the "SpatioTemporal RoPE" section of the HorizonStream
// post, with three axes).  Angles use the coordinate relative to the volume's
// origin: every logit depends on coordinate differences only, so this changes no
// logit and keeps the fp32 angles small.
//
// k_rope_pool: one workgroup per (block, head group, volume).  The block's tokens are gathered
// from packed order (perm); Q and K are rotated in fp32 and written with V in
// canonical order [B, H, NC, Dp] (rows zero-padded to Dp, empty slots zero rows);
// the block means of the rotated K and of V over the tokens present ([B, H, nblkp,
// Dp], zero rows for empty and padding blocks) are summed in a fixed order from
// LDS, so results are bitwise reproducible and independent of the packing.
// k_rope_pool_rows does the same with every head in one workgroup where rows need no
// padding (below).  HBM bound: reads q, k, v once, writes the rotated Q, K and V once.
#include <cmath>

#include "layout.h"

namespace pack3d {
namespace {

constexpr int kChunk = 32;  // tokens staged in LDS at a time (32: six workgroups per CU fit)

__global__ void k_rope_table(float2* tab, int rows, int half, int gw, double base) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * half) return;
  const int c = i / half, k = i - c * half;
  const double theta = pow(base, -2.0 * (double)k / (double)gw);
  const double phi = (double)c * theta;
  tab[i] = make_float2((float)cos(phi), (float)sin(phi));
}

template <typename T, int V>
struct alignas(sizeof(T) * V) Vec {
  T v[V];
};

template <typename T>
__device__ inline float to_f(T x) { return (float)x; }
template <typename T>
__device__ inline T from_f(float x) { return (T)x; }

struct RopeArgs {
  const void* q; const void* k; const void* v;
  const int32_t* coords; const int32_t* perm; const int32_t* geom; const int32_t* voff; const int32_t* count;
  const float2* tab;
  void* qrot; void* krot; void* vr; void* kbar; void* vbar;
  int NC, H, D, Dp, nblk, nblkp, bvol, heads_per_group, holes;
  int pool;  // 0: windowed-only attention reads no block means, so none are formed
  int bz, by, bx;  // block shape: a canonical slot's position in the volume follows from it
  int64_t in_stride;  // elements between consecutive tokens of q, k, v
  int pos_mode, groups, gw, half, trows;  // rotation groups (see Dims)
};

// GROUPS rotation groups of the head dim (3 axial, 1 packed 1D); ROTATE false: copy only.
template <typename T, int VEC, int GROUPS, bool ROTATE>
__global__ __launch_bounds__(256) void k_rope_pool(RopeArgs a) {
  extern __shared__ char smem[];
  const int blk = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int NC = a.NC, H = a.H, D = a.D, Dp = a.Dp, bvol = a.bvol;
  const int gw = D / GROUPS, half = gw / 2;
  constexpr int groups = GROUPS;
  const int ntok = bvol < kChunk ? bvol : kChunk;  // rows of the staging tiles
  const int nchunk = (bvol + kChunk - 1) / kChunk;   // the last chunk may be partial (|b| = 40, 48, 56)
  const bool pool = a.pool != 0;
  // LDS: src[bvol], rel[bvol][3] (int), kl[ntok][Dp+1], vl[ntok][Dp+1] (the input dtype: the
  // rotated K as stored, and V, are what the block means average)
  int* s_src = (int*)smem;
  int* s_rel = s_src + bvol;
  T* kl = (T*)(s_rel + 3 * bvol);
  const int ls = Dp + 1;
  T* vl = kl + ntok * ls;

  const int32_t* g = a.geom + b * G_FIELDS;
  const int64_t tok0 = a.voff[b];  // packed token offset of the volume
  // Axial angle rows: a canonical slot is block blk, offset t inside it, so its position
  // relative to the volume's origin is beta(blk) * b + w(t), the coordinate minus the origin
  // the index placed there (no gather of the coordinates).
  int base[3] = {0, 0, 0};
  if (GROUPS == 3) {
    const int nby = (g[G_EY] + a.by - 1) / a.by, nbx = (g[G_EX] + a.bx - 1) / a.bx;
    base[0] = blk / (nby * nbx) * a.bz;
    base[1] = (blk / nbx) % nby * a.by;
    base[2] = blk % nbx * a.bx;
  }
  for (int t = tid; t < bvol; t += 256) {
    const int kappa = blk * bvol + t;
    const int src = a.perm[(int64_t)b * NC + kappa];  // -1: empty slot
    s_src[t] = src;
    int rel[3] = {0, 0, 0};
    if (src >= 0 && ROTATE) {
      if (GROUPS == 3) {
        rel[0] = base[0] + t / (a.by * a.bx);
        rel[1] = base[1] + (t / a.bx) % a.by;
        rel[2] = base[2] + t % a.bx;
      } else {
        rel[0] = src;  // packed 1D: the position in the volume
      }
    }
    for (int gi = 0; gi < GROUPS; ++gi) {
      const int r = rel[gi];
      s_rel[t * 3 + gi] = r < 0 ? 0 : (r >= a.trows ? a.trows - 1 : r);
    }
  }
  __syncthreads();

  const T* q = (const T*)a.q;
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  T* qrot = (T*)a.qrot;
  T* krot = (T*)a.krot;
  T* vr = (T*)a.vr;
  const int pchunks = half / VEC;         // VEC-wide pieces per half group
  const int h0 = hg * a.heads_per_group;

  for (int hh = 0; hh < a.heads_per_group; ++hh) {
    const int h = h0 + hh;
    const int64_t bh = (int64_t)b * H + h;
    float csum = 0.f;   // K~ column tid (tid < Dp) or V column tid - Dp (tid < 2 Dp)
    for (int ch = 0; ch < nchunk; ++ch) {
      const int t0 = ch * kChunk;
      const int cnt = bvol - t0 < kChunk ? bvol - t0 : kChunk;  // tokens of this chunk
      const int rope_items = cnt * groups * pchunks;
      const int v_items = cnt * (D / VEC);
      // rotate q and k
      for (int it = tid; it < rope_items; it += 256) {
        const int tok = it / (groups * pchunks);
        const int rem = it - tok * groups * pchunks;
        const int ax = rem / pchunks, p = rem - ax * pchunks;  // group, pair chunk
        const int src = s_src[t0 + tok];
        const int c = s_rel[(t0 + tok) * 3 + ax];
        const int col1 = ax * gw + p * VEC, col2 = col1 + half;
        Vec<T, VEC> q1, q2, k1, k2;
        if (src >= 0) {
          const int64_t in_row = (tok0 + src) * a.in_stride + (int64_t)h * D;
          q1 = *(const Vec<T, VEC>*)(q + in_row + col1);
          q2 = *(const Vec<T, VEC>*)(q + in_row + col2);
          k1 = *(const Vec<T, VEC>*)(k + in_row + col1);
          k2 = *(const Vec<T, VEC>*)(k + in_row + col2);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) q1.v[e] = q2.v[e] = k1.v[e] = k2.v[e] = from_f<T>(0.f);
        }
        Vec<T, VEC> oq1, oq2, ok1, ok2;
        const float2* cs = a.tab + (int64_t)c * half + p * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          // no rotation: the identity row (cos 1, sin 0), and x2 * 0 must not turn inf into NaN
          const float2 r = ROTATE ? cs[e] : make_float2(1.f, 0.f);
          const float x1 = to_f(q1.v[e]), x2 = to_f(q2.v[e]);
          oq1.v[e] = ROTATE ? from_f<T>(x1 * r.x - x2 * r.y) : q1.v[e];
          oq2.v[e] = ROTATE ? from_f<T>(x1 * r.y + x2 * r.x) : q2.v[e];
          const float y1 = to_f(k1.v[e]), y2 = to_f(k2.v[e]);
          const float ky1 = ROTATE ? y1 * r.x - y2 * r.y : y1;
          const float ky2 = ROTATE ? y1 * r.y + y2 * r.x : y2;
          ok1.v[e] = from_f<T>(ky1);
          ok2.v[e] = from_f<T>(ky2);
          if (pool) {
            kl[tok * ls + col1 + e] = ok1.v[e];
            kl[tok * ls + col2 + e] = ok2.v[e];
          }
        }
        const int64_t out_row = (bh * NC + (int64_t)blk * bvol + t0 + tok) * Dp;
        *(Vec<T, VEC>*)(qrot + out_row + col1) = oq1;
        *(Vec<T, VEC>*)(qrot + out_row + col2) = oq2;
        *(Vec<T, VEC>*)(krot + out_row + col1) = ok1;
        *(Vec<T, VEC>*)(krot + out_row + col2) = ok2;
      }
      // copy v to canonical order
      for (int it = tid; it < v_items; it += 256) {
        const int tok = it / (D / VEC);
        const int col = (it - tok * (D / VEC)) * VEC;
        const int src = s_src[t0 + tok];
        Vec<T, VEC> x;
        if (src >= 0) {
          x = *(const Vec<T, VEC>*)(v + (tok0 + src) * a.in_stride + (int64_t)h * D + col);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) x.v[e] = from_f<T>(0.f);
        }
        *(Vec<T, VEC>*)(vr + (bh * NC + (int64_t)blk * bvol + t0 + tok) * Dp + col) = x;
        if (pool) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) vl[tok * ls + col + e] = x.v[e];
        }
      }
      // zero padding columns D..Dp of the rows and of the staged tiles
      if (Dp > D) {
        const int pad = Dp - D;
        for (int it = tid; it < cnt * pad; it += 256) {
          const int tok = it / pad, col = D + it - tok * pad;
          const int64_t out_row = (bh * NC + (int64_t)blk * bvol + t0 + tok) * Dp;
          qrot[out_row + col] = from_f<T>(0.f);
          krot[out_row + col] = from_f<T>(0.f);
          vr[out_row + col] = from_f<T>(0.f);
          if (pool) {
            kl[tok * ls + col] = from_f<T>(0.f);
            vl[tok * ls + col] = from_f<T>(0.f);
          }
        }
      }
      if (!pool) continue;  // no LDS staging to read back: the next chunk needs no barrier
      __syncthreads();
      // column sums over the chunk: threads 0 .. Dp-1 sum K~ columns, Dp .. 2Dp-1 V columns
      if (tid < 2 * Dp) {
        const T* col = tid < Dp ? kl + tid : vl + (tid - Dp);
        float cs = 0.f;
        for (int t = 0; t < cnt; ++t) cs += to_f(col[t * ls]);
        csum += cs;
      }
      __syncthreads();
    }
    if (pool && tid < 2 * Dp) {
      // mean over the tokens present (|b| on a full grid); an empty block's sums are 0
      const int cnt = a.holes ? a.count[(int64_t)b * a.nblk + blk] : bvol;
      const float inv = cnt > 0 ? 1.0f / (float)cnt : 0.f;
      T* bar = tid < Dp ? (T*)a.kbar : (T*)a.vbar;
      const int c = tid < Dp ? tid : tid - Dp;
      bar[(bh * a.nblkp + blk) * Dp + c] = from_f<T>(csum * inv);
      // zero the padding summaries nblk .. nblkp (there may be more of them than blocks)
      for (int pad_blk = a.nblk + blk; pad_blk < a.nblkp; pad_blk += a.nblk)
        bar[(bh * a.nblkp + pad_blk) * Dp + c] = from_f<T>(0.f);
    }
  }
}

// The same pass with all heads in one workgroup, for rows without padding (Dp = D) whose
// rotation pairs fall in whole 16-byte pieces.  One workgroup per (block, volume); a row
// group of P threads covers one token's q, k and v rows whole (H * D contiguous elements
// each in the packed input), each thread one rotation pair of VEC-element pieces of one
// head, so every token's rows are read as full aligned runs.  A thread keeps the column
// sums of its K~ and V pieces over the tokens of its row group; the R row groups' sums are
// then added in a fixed order through LDS, so the block means stay bitwise reproducible
// and independent of the packing.
template <typename T, int GROUPS, bool ROTATE>
__global__ __launch_bounds__(256) void k_rope_pool_rows(RopeArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  extern __shared__ char smem[];
  const int blk = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int NC = a.NC, H = a.H, D = a.D, bvol = a.bvol;
  const int gw = D / GROUPS, half = gw / 2, pchunks = half / VEC;
  const int per_head = D / (2 * VEC);  // rotation-pair items per head
  const int P = H * per_head;          // threads per row group (host: P <= 256)
  const int R = 256 / P;               // row groups
  const int r = tid / P, pi = tid - r * P;
  const bool pool = a.pool != 0;
  // LDS: src[bvol], rel[bvol][3] (int), then the partial sums [4 VEC][256] (float)
  int* s_src = (int*)smem;
  int* s_rel = s_src + bvol;
  float* s_sum = (float*)(s_rel + 3 * bvol);

  const int32_t* g = a.geom + b * G_FIELDS;
  const int64_t tok0 = a.voff[b];
  int base[3] = {0, 0, 0};
  if (GROUPS == 3) {
    const int nby = (g[G_EY] + a.by - 1) / a.by, nbx = (g[G_EX] + a.bx - 1) / a.bx;
    base[0] = blk / (nby * nbx) * a.bz;
    base[1] = (blk / nbx) % nby * a.by;
    base[2] = blk % nbx * a.bx;
  }
  for (int t = tid; t < bvol; t += 256) {
    const int src = a.perm[(int64_t)b * NC + blk * bvol + t];  // -1: empty slot
    s_src[t] = src;
    int rel[3] = {0, 0, 0};
    if (src >= 0 && ROTATE) {
      if (GROUPS == 3) {
        rel[0] = base[0] + t / (a.by * a.bx);
        rel[1] = base[1] + (t / a.bx) % a.by;
        rel[2] = base[2] + t % a.bx;
      } else {
        rel[0] = src;
      }
    }
    for (int gi = 0; gi < GROUPS; ++gi) {
      const int rr = rel[gi];
      s_rel[t * 3 + gi] = rr < 0 ? 0 : (rr >= a.trows ? a.trows - 1 : rr);
    }
  }
  __syncthreads();

  const int h = pi / per_head, j = pi - h * per_head;
  const int ax = j / pchunks, p = j - ax * pchunks;
  const int col1 = ax * gw + p * VEC, col2 = col1 + half;
  float ks1[VEC], ks2[VEC], vs1[VEC], vs2[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) ks1[e] = ks2[e] = vs1[e] = vs2[e] = 0.f;
  if (r < R) {
    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    const int64_t orow0 = ((int64_t)b * H + h) * NC + (int64_t)blk * bvol;
    // two tokens per trip, both tokens' loads issued before either is stored
    auto load = [&](int t, Vec<T, VEC> (&x)[6]) {
      const int src = s_src[t];
      if (src >= 0) {
        const int64_t in_row = (tok0 + src) * a.in_stride + (int64_t)h * D;
        x[0] = *(const Vec<T, VEC>*)(q + in_row + col1);
        x[1] = *(const Vec<T, VEC>*)(q + in_row + col2);
        x[2] = *(const Vec<T, VEC>*)(k + in_row + col1);
        x[3] = *(const Vec<T, VEC>*)(k + in_row + col2);
        x[4] = *(const Vec<T, VEC>*)(v + in_row + col1);
        x[5] = *(const Vec<T, VEC>*)(v + in_row + col2);
      } else {
#pragma unroll
        for (int i = 0; i < 6; ++i)
#pragma unroll
          for (int e = 0; e < VEC; ++e) x[i].v[e] = from_f<T>(0.f);
      }
    };
    auto store = [&](int t, const Vec<T, VEC> (&x)[6]) {
      const float2* cs = a.tab + (int64_t)s_rel[t * 3 + ax] * half + p * VEC;
      Vec<T, VEC> oq1, oq2, ok1, ok2;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        // each rotated value as one product rounded, then a fused multiply-add, so the bits
        // do not depend on how the compiler contracts the expression
        const float2 rot = ROTATE ? cs[e] : make_float2(1.f, 0.f);
        const float x1 = to_f(x[0].v[e]), x2 = to_f(x[1].v[e]);
        oq1.v[e] = ROTATE ? from_f<T>(fmaf(x1, rot.x, -(x2 * rot.y))) : x[0].v[e];
        oq2.v[e] = ROTATE ? from_f<T>(fmaf(x1, rot.y, x2 * rot.x)) : x[1].v[e];
        const float y1 = to_f(x[2].v[e]), y2 = to_f(x[3].v[e]);
        ok1.v[e] = ROTATE ? from_f<T>(fmaf(y1, rot.x, -(y2 * rot.y))) : x[2].v[e];
        ok2.v[e] = ROTATE ? from_f<T>(fmaf(y1, rot.y, y2 * rot.x)) : x[3].v[e];
        // the block means average the rotated K as stored, and V
        ks1[e] += to_f(ok1.v[e]);
        ks2[e] += to_f(ok2.v[e]);
        vs1[e] += to_f(x[4].v[e]);
        vs2[e] += to_f(x[5].v[e]);
      }
      const int64_t out_row = (orow0 + t) * D;
      *(Vec<T, VEC>*)((T*)a.qrot + out_row + col1) = oq1;
      *(Vec<T, VEC>*)((T*)a.qrot + out_row + col2) = oq2;
      *(Vec<T, VEC>*)((T*)a.krot + out_row + col1) = ok1;
      *(Vec<T, VEC>*)((T*)a.krot + out_row + col2) = ok2;
      *(Vec<T, VEC>*)((T*)a.vr + out_row + col1) = x[4];
      *(Vec<T, VEC>*)((T*)a.vr + out_row + col2) = x[5];
    };
    for (int t = r; t < bvol; t += 2 * R) {
      Vec<T, VEC> xa[6], xb[6];
      const bool two = t + R < bvol;
      load(t, xa);
      if (two) load(t + R, xb);
      store(t, xa);
      if (two) store(t + R, xb);
    }
  }
  if (!pool) return;
  // partial sums [e][tid] (e: K~ piece 1, K~ piece 2, V piece 1, V piece 2, VEC each)
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    s_sum[(0 * VEC + e) * 256 + tid] = ks1[e];
    s_sum[(1 * VEC + e) * 256 + tid] = ks2[e];
    s_sum[(2 * VEC + e) * 256 + tid] = vs1[e];
    s_sum[(3 * VEC + e) * 256 + tid] = vs2[e];
  }
  __syncthreads();
  // mean over the tokens present (|b| on a full grid); an empty block's sums are 0
  const int cnt = a.holes ? a.count[(int64_t)b * a.nblk + blk] : bvol;
  const float inv = cnt > 0 ? 1.0f / (float)cnt : 0.f;
  for (int it = tid; it < 4 * VEC * P; it += 256) {
    const int e4 = it / P, qi = it - e4 * P;  // piece element, pair item
    float sum = 0.f;
    for (int rr = 0; rr < R; ++rr) sum += s_sum[e4 * 256 + rr * P + qi];  // row groups in order
    const int hh = qi / per_head, jj = qi - hh * per_head;
    const int aa = jj / pchunks, pp = jj - aa * pchunks;
    const int which = e4 / VEC, el = e4 - which * VEC;
    const int c = aa * gw + pp * VEC + (which & 1 ? half : 0) + el;
    T* bar = which < 2 ? (T*)a.kbar : (T*)a.vbar;
    const int64_t brow = ((int64_t)b * H + hh) * a.nblkp;
    bar[(brow + blk) * D + c] = from_f<T>(sum * inv);
    // zero the padding summaries nblk .. nblkp (there may be more of them than blocks)
    for (int pad_blk = a.nblk + blk; pad_blk < a.nblkp; pad_blk += a.nblk) bar[(brow + pad_blk) * D + c] = from_f<T>(0.f);
  }
}

// Threads of one row group of k_rope_pool_rows (0: the layout does not suit it).
inline int rows_kernel_threads(const Dims& d) {
  const int vec = 16 / (int)d.esize;
  if (d.Dp != d.D || d.half % vec != 0) return 0;
  const int p = d.H * d.D / (2 * vec);
  return p <= 256 ? p : 0;
}

template <typename T, int GROUPS, bool ROTATE>
void launch_mode(const Dims& d, const RopeArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  int vec = 1;
  const int cap = 16 / (int)sizeof(T);
  while (vec * 2 <= cap && d.half % (vec * 2) == 0) vec *= 2;
  switch (vec) {
    case 1: hipLaunchKernelGGL((k_rope_pool<T, 1, GROUPS, ROTATE>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_rope_pool<T, 2, GROUPS, ROTATE>), grid, dim3(256), lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_rope_pool<T, 4, GROUPS, ROTATE>), grid, dim3(256), lds, s, a); break;
    default:
      if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((k_rope_pool<T, 8, GROUPS, ROTATE>), grid, dim3(256), lds, s, a);
      break;
  }
}

template <typename T>
pack3d_status launch_typed(const Dims& d, const RopeArgs& a, const char* name, hipStream_t s) {
  if (rows_kernel_threads(d) > 0) {
    const size_t lds = sizeof(int) * 4 * d.bvol + (a.pool ? sizeof(float) * 4 * (16 / sizeof(T)) * 256 : 0);
    const dim3 grid(d.nblk, 1, d.B);
    ProfileScope prof(name, s);
    if (d.pos_mode == PACK3D_POS_AXIAL) hipLaunchKernelGGL((k_rope_pool_rows<T, 3, true>), grid, dim3(256), lds, s, a);
    else if (d.pos_mode == PACK3D_POS_PACKED_1D) hipLaunchKernelGGL((k_rope_pool_rows<T, 1, true>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((k_rope_pool_rows<T, 1, false>), grid, dim3(256), lds, s, a);
    return check_launch("rope/pool");
  }
  const int ntok = d.bvol < kChunk ? d.bvol : kChunk;
  // the staging tiles exist only to form the block means
  const size_t lds = sizeof(int) * 4 * d.bvol + (a.pool ? 2 * sizeof(T) * ntok * (d.Dp + 1) : 0);
  dim3 grid(d.nblk, d.H / a.heads_per_group, d.B);
  ProfileScope prof(name, s);
  if (d.pos_mode == PACK3D_POS_AXIAL) launch_mode<T, 3, true>(d, a, grid, lds, s);
  else if (d.pos_mode == PACK3D_POS_PACKED_1D) launch_mode<T, 1, true>(d, a, grid, lds, s);
  else launch_mode<T, 1, false>(d, a, grid, lds, s);
  return check_launch("rope/pool");
}

}  // namespace

pack3d_status launch_rope_pool(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                               const void* q, const void* k, const void* v, const int32_t* coords,
                               char* ws, const Workspace& w, const char* name, hipStream_t s) {
  const int n_tab = d.trows * d.half;
  {
    ProfileScope prof("rope_table", s);
    hipLaunchKernelGGL(k_rope_table, dim3((n_tab + 255) / 256), dim3(256), 0, s,
                       (float2*)(ws + w.rope), d.trows, d.half, d.gw, (double)at->rope_base);
  }
  RopeArgs a;
  a.q = q; a.k = k; a.v = v; a.coords = coords; a.perm = ix->perm; a.geom = ix->geom;
  a.voff = ix->voff; a.count = ix->count; a.holes = d.holes;
  a.tab = (const float2*)(ws + w.rope);
  a.qrot = ws + w.qrot; a.krot = ws + w.krot; a.vr = ws + w.vr; a.kbar = ws + w.kbar; a.vbar = ws + w.vbar;
  a.in_stride = d.in_stride;
  a.pool = at->with_summaries ? 1 : 0;
  a.bz = ix->block[0]; a.by = ix->block[1]; a.bx = ix->block[2];
  a.NC = d.NC; a.H = d.H; a.D = d.D; a.Dp = d.Dp; a.nblk = d.nblk; a.nblkp = d.nblkp; a.bvol = d.bvol;
  a.pos_mode = d.pos_mode; a.groups = d.groups; a.gw = d.gw; a.half = d.half; a.trows = d.trows;
  // heads per workgroup: the fewest whose rows cover whole 128-byte lines, else all
  int hp = d.H;
  for (int c = 1; c <= d.H; ++c) {
    if (d.H % c == 0 && ((size_t)c * d.D * d.esize) % 128 == 0) { hp = c; break; }
  }
  a.heads_per_group = hp;
  return at->dtype == PACK3D_BF16 ? launch_typed<bf16>(d, a, name, s) : launch_typed<float>(d, a, name, s);
}

}  // namespace pack3d
