// K0: index builder -- block membership, canonical order and neighbour table of
// each packed volume, derived from the tokens' true (z, y, x) grid coordinates.
//
// "Geometry Matters in Packed 3D Attention" (abstract): the operator separates the
// memory layout from the attention geometry, so every table here is a function of
// the coordinates alone; the packing order only decides where each token's entry
// is stored.  Readings: the block lattice is anchored at each volume's componentwise
// minimum coordinate; the local set is block-granular (Chebyshev radius r in block
// units).  Without the ragged flag only full grids whose extents divide by the block
// are accepted; with it a volume is any set of distinct points, covered by
// ceil(extent / b) blocks per axis, and canonical slots without a token stay empty.
//
// Kernels (all integer, exact):
//   init      geom <- sentinels
//   extents   per-volume componentwise min / max (atomicMin / atomicMax)
//   check     per-volume extents, block count and status
//   clear     perm <- INT_MAX, count <- 0
//   assign    per token: block id, canonical slot, atomicMin(perm[slot], token), count
//   dups      per token: perm[slot] != token -> duplicate; lowest such token kept
//   finish    perm INT_MAX -> -1; occupancy bits of the slots; empty-block bits
//   nbr       per (volume, block, slot): neighbour id or -1
#include <climits>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "layout.h"

namespace pack3d {
namespace {

__global__ void k_init(int32_t* geom, int32_t batch) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= batch * G_FIELDS) return;
  const int f = i % G_FIELDS;
  int32_t v = 0;
  if (f <= G_OX) v = INT_MAX;                      // running minimum
  else if (f <= G_EX) v = INT_MIN;                 // running maximum (turned into extent later)
  else if (f == G_STATUS) v = GS_OK;
  else if (f == G_TOKEN) v = INT_MAX;              // offending token (minimum)
  geom[i] = v;
}

// One thread per token (grid.y = volume); wave-level reduction before the atomics.
__global__ void k_extents(const int32_t* __restrict__ coords, const int32_t* __restrict__ voff, int32_t* geom) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t n = voff[vol + 1] - voff[vol];
  int32_t mn[3] = {INT_MAX, INT_MAX, INT_MAX}, mx[3] = {INT_MIN, INT_MIN, INT_MIN};
  if (i < n) {
    const int32_t* c = coords + ((int64_t)voff[vol] + i) * 3;
    for (int a = 0; a < 3; ++a) mn[a] = mx[a] = c[a];
  }
  for (int a = 0; a < 3; ++a) {
    for (int off = 32; off > 0; off >>= 1) {
      mn[a] = min(mn[a], __shfl_xor(mn[a], off));
      mx[a] = max(mx[a], __shfl_xor(mx[a], off));
    }
  }
  if ((threadIdx.x & 63) == 0 && (int32_t)(blockIdx.x * blockDim.x + (threadIdx.x & ~63)) < n) {
    int32_t* g = geom + vol * G_FIELDS;
    for (int a = 0; a < 3; ++a) {
      atomicMin(g + G_OZ + a, mn[a]);
      atomicMax(g + G_EZ + a, mx[a]);
    }
  }
}

struct BlockShape { int32_t bz, by, bx, bvol; };

// One thread per volume: max -> extent, block count, then validate the grid.
__global__ void k_check(int32_t* geom, const int32_t* __restrict__ voff, int32_t batch, BlockShape b,
                        int32_t ragged, int32_t max_blocks) {
  const int32_t vol = blockIdx.x * blockDim.x + threadIdx.x;
  if (vol >= batch) return;
  int32_t* g = geom + vol * G_FIELDS;
  const int32_t n = voff[vol + 1] - voff[vol];
  g[G_NTOK] = n;
  if (n <= 0) {
    for (int a = 0; a < 3; ++a) g[G_OZ + a] = g[G_EZ + a] = 0;
    g[G_NBLK] = 0;
    g[G_STATUS] = GS_EMPTY;
    return;
  }
  int64_t e[3];
  for (int a = 0; a < 3; ++a) e[a] = (int64_t)g[G_EZ + a] - (int64_t)g[G_OZ + a] + 1;
  const int32_t bs[3] = {b.bz, b.by, b.bx};
  int64_t nb[3], nblk = 1;
  for (int a = 0; a < 3; ++a) {
    nb[a] = (e[a] + bs[a] - 1) / bs[a];
    nblk = nblk * nb[a] > ((int64_t)1 << 40) ? ((int64_t)1 << 40) : nblk * nb[a];
  }
  int status = GS_OK;
  if (!ragged) {
    // product of extents == n, computed without overflow (each extent <= n first)
    if (e[0] > n || e[1] > n || e[2] > n) status = GS_GRID;
    else if (e[0] * e[1] > n || e[0] * e[1] * e[2] != n) status = GS_GRID;
    else if (e[0] % b.bz || e[1] % b.by || e[2] % b.bx) status = GS_DIVISIBLE;
  }
  if (status == GS_OK && nblk > max_blocks) status = GS_BLOCKS;
  for (int a = 0; a < 3; ++a) g[G_EZ + a] = (int32_t)(e[a] > INT_MAX ? INT_MAX : e[a]);
  g[G_NBLK] = (int32_t)(nblk > INT_MAX ? INT_MAX : nblk);
  g[G_STATUS] = status;
}

__global__ void k_clear(int32_t* perm, int64_t nperm, int32_t* count, int64_t ncount) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nperm) perm[i] = INT_MAX;
  if (i < ncount) count[i] = 0;
}

__device__ inline int32_t blocks_along(const int32_t* g, int a, int32_t b) { return (g[G_EZ + a] + b - 1) / b; }

__global__ void k_assign(const int32_t* __restrict__ coords, const int32_t* __restrict__ voff,
                         const int32_t* __restrict__ geom, int32_t* token_block, int32_t* canon, int32_t* perm,
                         int32_t* count, int32_t nc, int32_t nblk, BlockShape b) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t n = voff[vol + 1] - voff[vol];
  if (i >= n) return;
  const int32_t* g = geom + vol * G_FIELDS;
  const int64_t t = (int64_t)voff[vol] + i;
  if (g[G_STATUS] != GS_OK) {
    token_block[t] = -1;
    canon[t] = -1;
    return;
  }
  const int32_t* c = coords + t * 3;
  const int32_t rz = c[0] - g[G_OZ], ry = c[1] - g[G_OY], rx = c[2] - g[G_OX];
  const int32_t nby = blocks_along(g, 1, b.by), nbx = blocks_along(g, 2, b.bx);
  const int32_t qz = rz / b.bz, qy = ry / b.by, qx = rx / b.bx;   // in range: rz .. rx >= 0
  const int32_t blk = (qz * nby + qy) * nbx + qx;
  const int32_t w = ((rz - qz * b.bz) * b.by + (ry - qy * b.by)) * b.bx + (rx - qx * b.bx);
  const int32_t slot = blk * b.bvol + w;
  token_block[t] = blk;
  canon[t] = slot;
  atomicMin(perm + (int64_t)vol * nc + slot, i);
  atomicAdd(count + (int64_t)vol * nblk + blk, 1);
}

__global__ void k_dups(const int32_t* __restrict__ canon, const int32_t* __restrict__ voff,
                       const int32_t* __restrict__ perm, int32_t* geom, int32_t nc) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t n = voff[vol + 1] - voff[vol];
  if (i >= n) return;
  int32_t* g = geom + vol * G_FIELDS;
  if (g[G_STATUS] != GS_OK && g[G_STATUS] != GS_DUPLICATE) return;
  const int32_t s = canon[(int64_t)voff[vol] + i];
  if (s < 0) return;
  if (perm[(int64_t)vol * nc + s] != i) {
    atomicMin(g + G_TOKEN, i);
    g[G_STATUS] = GS_DUPLICATE;  // every writer stores the same value
  }
}

// One thread per 32-slot word: INT_MAX -> -1 and the occupancy word; one thread per
// 32-block word of the empty-block mask (blocks past the volume's own count are empty).
__global__ void k_finish(int32_t* perm, uint32_t* occ, const int32_t* __restrict__ count, uint32_t* emask,
                         int32_t nc, int32_t occ_words, int32_t nblk, int32_t mask_words) {
  const int32_t vol = blockIdx.y;
  const int32_t w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w < occ_words) {
    uint32_t bits = 0u;
    for (int j = 0; j < 32; ++j) {
      const int32_t slot = w * 32 + j;
      if (slot >= nc) break;
      int32_t* p = perm + (int64_t)vol * nc + slot;
      if (*p == INT_MAX) *p = -1;
      else bits |= 1u << j;
    }
    occ[(int64_t)vol * occ_words + w] = bits;
  }
  if (w < mask_words) {
    uint32_t bits = 0u;
    for (int j = 0; j < 32; ++j) {
      const int32_t blk = w * 32 + j;
      if (blk >= nblk || count[(int64_t)vol * nblk + blk] == 0) bits |= 1u << j;
    }
    emask[(int64_t)vol * mask_words + w] = bits;
  }
}

__global__ void k_nbr(const int32_t* __restrict__ geom, int32_t* nbr, int32_t nblk, int32_t radius,
                      BlockShape b) {
  const int32_t vol = blockIdx.y;
  const int32_t span = 2 * radius + 1;
  const int32_t slots = span * span * span;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nblk * slots) return;
  const int32_t* g = geom + vol * G_FIELDS;
  int32_t* out = nbr + (int64_t)vol * nblk * slots;
  const int32_t blk = (int32_t)(i / slots), s = (int32_t)(i % slots);
  if (g[G_STATUS] != GS_OK || blk >= g[G_NBLK]) { out[i] = -1; return; }
  const int32_t nbz = blocks_along(g, 0, b.bz), nby = blocks_along(g, 1, b.by), nbx = blocks_along(g, 2, b.bx);
  const int32_t z = blk / (nby * nbx), y = (blk / nbx) % nby, x = blk % nbx;
  const int32_t dz = s / (span * span) - radius, dy = (s / span) % span - radius, dx = s % span - radius;
  const int32_t zz = z + dz, yy = y + dy, xx = x + dx;
  const bool in = zz >= 0 && zz < nbz && yy >= 0 && yy < nby && xx >= 0 && xx < nbx;
  out[i] = in ? (zz * nby + yy) * nbx + xx : -1;
}

struct TableLayout {
  size_t geom, voff, token_block, canon, perm, nbr, count, occ, emask, total;
  int32_t nc, occ_words, mask_words;
};

TableLayout table_layout(int32_t batch, int64_t total, int32_t nblk, int32_t bvol, int32_t slots) {
  TableLayout t;
  t.nc = nblk * bvol;
  t.occ_words = (t.nc + 31) / 32;
  t.mask_words = (nblk + kTile - 1) / kTile * kTile / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  t.geom = take(sizeof(int32_t) * batch * G_FIELDS);
  t.voff = take(sizeof(int32_t) * (batch + 1));
  t.token_block = take(sizeof(int32_t) * (size_t)total);
  t.canon = take(sizeof(int32_t) * (size_t)total);
  t.perm = take(sizeof(int32_t) * (size_t)batch * t.nc);
  t.nbr = take(sizeof(int32_t) * (size_t)batch * nblk * slots);
  t.count = take(sizeof(int32_t) * (size_t)batch * nblk);
  t.occ = take(sizeof(uint32_t) * (size_t)batch * t.occ_words);
  t.emask = take(sizeof(uint32_t) * (size_t)batch * t.mask_words);
  t.total = off;
  return t;
}

// Host view of the batch layout: offsets of every volume, checked.
struct Layout {
  int32_t batch, nmax;
  int64_t total;
  const int32_t* off;   // caller's offsets or nullptr (uniform)
  int32_t n;            // uniform tokens per volume
  int32_t tokens(int v) const { return off ? off[v + 1] - off[v] : n; }
  int64_t start(int v) const { return off ? off[v] : (int64_t)v * n; }
};

pack3d_status read_layout(const pack3d_packing* p, const char* who, Layout& L) {
  if (!p) return set_error(PACK3D_E_INVALID, "%s: null packing", who);
  if (p->batch < 1) return set_error(PACK3D_E_INVALID, "%s: batch must be >= 1", who);
  if (p->ragged != 0 && p->ragged != 1) return set_error(PACK3D_E_INVALID, "%s: ragged must be 0 or 1", who);
  L.batch = p->batch;
  L.off = p->volume_offsets;
  L.n = p->tokens_per_volume;
  if (!L.off) {
    if (p->tokens_per_volume < 1) return set_error(PACK3D_E_INVALID, "%s: tokens_per_volume must be >= 1", who);
    L.total = (int64_t)p->batch * p->tokens_per_volume;
    L.nmax = p->tokens_per_volume;
  } else {
    if (L.off[0] != 0) return set_error(PACK3D_E_INVALID, "%s: volume_offsets[0] must be 0", who);
    L.nmax = 0;
    for (int v = 0; v < p->batch; ++v) {
      const int32_t n = L.off[v + 1] - L.off[v];
      if (L.off[v + 1] < L.off[v] || n < 1)
        return set_error(PACK3D_E_INVALID, "%s: volume %d has no tokens (offsets must increase)", who, v);
      L.nmax = n > L.nmax ? n : L.nmax;
    }
    L.total = L.off[p->batch];
  }
  if (L.total > INT32_MAX) return set_error(PACK3D_E_UNSUPPORTED, "%s: more than 2^31 - 1 tokens", who);
  return PACK3D_OK;
}

pack3d_status check_block(const int32_t* block, int32_t r, const char* who) {
  if (!block || block[0] < 1 || block[1] < 1 || block[2] < 1)
    return set_error(PACK3D_E_INVALID, "%s: block extents must be >= 1", who);
  if (r < 0) return set_error(PACK3D_E_INVALID, "%s: radius must be >= 0", who);
  if (r > 7) return set_error(PACK3D_E_UNSUPPORTED, "%s: local_radius %d > 7 is not supported", who, r);
  const int64_t bvol = (int64_t)block[0] * block[1] * block[2];
  if (bvol % 8)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: block volume %lld is not a multiple of 8", who, (long long)bvol);
  if (bvol > 64 && bvol % 64)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: block volume %lld above 64 must be a multiple of 64", who,
                     (long long)bvol);
  if (bvol > kMaxBlockTokens)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: %lld tokens per block > %d", who, (long long)bvol, kMaxBlockTokens);
  return PACK3D_OK;
}

// Blocks per volume the tables hold: N_v / |b| (largest) without ragged, max_blocks with it.
pack3d_status table_blocks(const pack3d_packing* p, const Layout& L, int32_t bvol, const char* who, int32_t& nblk) {
  if (p->ragged) {
    if (p->max_blocks < 1) return set_error(PACK3D_E_INVALID, "%s: ragged packing needs max_blocks >= 1", who);
    nblk = p->max_blocks;
  } else {
    for (int v = 0; v < L.batch; ++v)
      if (L.tokens(v) % bvol)
        return set_error(PACK3D_E_COORDS, "%s: volume %d: %d tokens cannot tile into %d-token blocks", who, v,
                         L.tokens(v), bvol);
    nblk = L.nmax / bvol;
  }
  if ((int64_t)nblk * bvol > INT32_MAX / 2)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: %d blocks of %d tokens per volume is too large", who, nblk, bvol);
  return PACK3D_OK;
}

// geometry record errors -> status + message (volume v)
pack3d_status geometry_error(const int32_t* g, int v, const BlockShape& b, int32_t max_blocks) {
  switch (g[G_STATUS]) {
    case GS_GRID:
      return set_error(PACK3D_E_COORDS, "build_index: volume %d: coordinates do not fill their bounding box "
                       "(extent %d x %d x %d for %d tokens)", v, g[G_EZ], g[G_EY], g[G_EX], g[G_NTOK]);
    case GS_DIVISIBLE:
      return set_error(PACK3D_E_COORDS, "build_index: volume %d: extent %d x %d x %d not divisible by block "
                       "%d x %d x %d", v, g[G_EZ], g[G_EY], g[G_EX], b.bz, b.by, b.bx);
    case GS_EMPTY:
      return set_error(PACK3D_E_COORDS, "build_index: volume %d has no tokens", v);
    case GS_BLOCKS:
      return set_error(PACK3D_E_COORDS, "build_index: volume %d needs %d blocks (extent %d x %d x %d), the tables "
                       "hold %d", v, g[G_NBLK], g[G_EZ], g[G_EY], g[G_EX], max_blocks);
    default:
      return set_error(PACK3D_E_COORDS, "build_index: volume %d: duplicate point at local index %d", v, g[G_TOKEN]);
  }
}

// Device offsets (in the caller's buffer) and the extent pass; geometry checked against
// max_blocks.  `off` is the host source of the copy: the caller keeps it alive until it
// has synchronized the stream.
pack3d_status launch_geometry(const int32_t* coords, const Layout& L, BlockShape b, int32_t ragged,
                              int32_t max_blocks, int32_t* geom, int32_t* voff, std::vector<int32_t>& off,
                              hipStream_t s) {
  const int threads = 256;
  off.resize(L.batch + 1);
  for (int v = 0; v <= L.batch; ++v) off[v] = (int32_t)(v < L.batch ? L.start(v) : L.total);
  hipError_t e = hipMemcpyAsync(voff, off.data(), sizeof(int32_t) * (L.batch + 1), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return set_error(PACK3D_E_HIP, "build_index: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(k_init, dim3((L.batch * G_FIELDS + threads - 1) / threads), dim3(threads), 0, s, geom, L.batch);
  dim3 tok_grid((unsigned)((L.nmax + threads - 1) / threads), (unsigned)L.batch);
  hipLaunchKernelGGL(k_extents, tok_grid, dim3(threads), 0, s, coords, voff, geom);
  hipLaunchKernelGGL(k_check, dim3((L.batch + 63) / 64), dim3(64), 0, s, geom, voff, L.batch, b, ragged, max_blocks);
  return check_launch("build_index: geometry");
}

pack3d_status read_geom(int32_t* host, const int32_t* geom, int32_t batch, hipStream_t s) {
  hipError_t e = hipMemcpyAsync(host, geom, sizeof(int32_t) * batch * G_FIELDS, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_error(PACK3D_E_HIP, "build_index: %s", hipGetErrorString(e));
  return PACK3D_OK;
}

}  // namespace
}  // namespace pack3d

using namespace pack3d;

extern "C" size_t pack3d_index_bytes(const pack3d_packing* packing, const int32_t block_shape[3],
                                     int32_t local_radius) {
  Layout L;
  if (read_layout(packing, "index_bytes", L) != PACK3D_OK) return 0;
  if (check_block(block_shape, local_radius, "index_bytes") != PACK3D_OK) return 0;
  const int32_t bvol = block_shape[0] * block_shape[1] * block_shape[2];
  int32_t nblk;
  if (table_blocks(packing, L, bvol, "index_bytes", nblk) != PACK3D_OK) return 0;
  const int32_t span = 2 * local_radius + 1;
  return table_layout(L.batch, L.total, nblk, bvol, span * span * span).total;
}

extern "C" pack3d_status pack3d_measure_blocks(const int32_t* coords_dev, const pack3d_packing* packing,
                                               const int32_t block_shape[3], void* scratch_dev,
                                               size_t scratch_bytes, void* stream, int32_t* max_blocks_out) {
  if (!coords_dev || !scratch_dev || !max_blocks_out)
    return set_error(PACK3D_E_INVALID, "measure_blocks: null pointer argument");
  Layout L;
  pack3d_status st = read_layout(packing, "measure_blocks", L);
  if (st != PACK3D_OK) return st;
  st = check_block(block_shape, 0, "measure_blocks");
  if (st != PACK3D_OK) return st;
  if (scratch_bytes < (size_t)64 * L.batch)
    return set_error(PACK3D_E_WORKSPACE, "measure_blocks: scratch %zu bytes < %zu needed", scratch_bytes,
                     (size_t)64 * L.batch);
  hipStream_t s = (hipStream_t)stream;
  int32_t* geom = (int32_t*)scratch_dev;
  int32_t* voff = geom + (size_t)L.batch * G_FIELDS;   // 40 B + 4 (B + 1) <= 64 B per volume
  const BlockShape b{block_shape[0], block_shape[1], block_shape[2], block_shape[0] * block_shape[1] * block_shape[2]};
  std::vector<int32_t> off;
  st = launch_geometry(coords_dev, L, b, 1, INT32_MAX, geom, voff, off, s);
  if (st != PACK3D_OK) {
    hipStreamSynchronize(s);
    return st;
  }
  std::vector<int32_t> hg((size_t)L.batch * G_FIELDS);
  st = read_geom(hg.data(), geom, L.batch, s);
  if (st != PACK3D_OK) return st;
  int32_t m = 0;
  for (int v = 0; v < L.batch; ++v) {
    const int32_t* g = hg.data() + (size_t)v * G_FIELDS;
    if (g[G_STATUS] == GS_EMPTY) return set_error(PACK3D_E_COORDS, "measure_blocks: volume %d has no tokens", v);
    m = g[G_NBLK] > m ? g[G_NBLK] : m;
  }
  *max_blocks_out = m;
  return PACK3D_OK;
}

extern "C" pack3d_status pack3d_build_index(const int32_t* coords_dev, const pack3d_packing* packing,
                                            const int32_t block_shape[3], int32_t local_radius,
                                            void* tables_dev, size_t tables_bytes, void* stream,
                                            pack3d_index** out) {
  if (out) *out = nullptr;
  if (!coords_dev || !tables_dev || !out)
    return set_error(PACK3D_E_INVALID, "build_index: null pointer argument");
  Layout L;
  pack3d_status st = read_layout(packing, "build_index", L);
  if (st != PACK3D_OK) return st;
  st = check_block(block_shape, local_radius, "build_index");
  if (st != PACK3D_OK) return st;
  const int32_t bvol = block_shape[0] * block_shape[1] * block_shape[2];
  int32_t cap;   // blocks per volume the tables hold
  st = table_blocks(packing, L, bvol, "build_index", cap);
  if (st != PACK3D_OK) return st;
  const int32_t span = 2 * local_radius + 1, slots = span * span * span;
  const TableLayout cap_layout = table_layout(L.batch, L.total, cap, bvol, slots);
  if (tables_bytes < cap_layout.total)
    return set_error(PACK3D_E_WORKSPACE, "build_index: tables buffer %zu bytes < %zu needed", tables_bytes,
                     cap_layout.total);

  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)tables_dev;
  int32_t* geom = (int32_t*)(base + cap_layout.geom);
  int32_t* voff = (int32_t*)(base + cap_layout.voff);
  const BlockShape b{block_shape[0], block_shape[1], block_shape[2], bvol};
  const int32_t ragged = packing->ragged;
  std::vector<int32_t> off;
  st = launch_geometry(coords_dev, L, b, ragged, cap, geom, voff, off, s);
  if (st != PACK3D_OK) {
    hipStreamSynchronize(s);
    return st;
  }

  int32_t* host_geom = (int32_t*)std::malloc(sizeof(int32_t) * L.batch * G_FIELDS);
  if (!host_geom) return set_error(PACK3D_E_INVALID, "build_index: host allocation failed");
  auto fail = [&](pack3d_status r) {
    std::free(host_geom);
    return r;
  };
  // Ragged: the block count comes from the coordinates, so read the geometry before laying
  // out the tables (compact to the largest actual count).  Otherwise it is N_v / |b|.
  int32_t nblk = cap;
  if (ragged) {
    st = read_geom(host_geom, geom, L.batch, s);
    if (st != PACK3D_OK) return fail(st);
    nblk = 1;
    for (int v = 0; v < L.batch; ++v) {
      const int32_t* g = host_geom + v * G_FIELDS;
      if (g[G_STATUS] != GS_OK) return fail(geometry_error(g, v, b, cap));
      nblk = g[G_NBLK] > nblk ? g[G_NBLK] : nblk;
    }
  }
  const TableLayout T = table_layout(L.batch, L.total, nblk, bvol, slots);   // geom and voff unmoved
  int32_t* token_block = (int32_t*)(base + T.token_block);
  int32_t* canon = (int32_t*)(base + T.canon);
  int32_t* perm = (int32_t*)(base + T.perm);
  int32_t* nbr = (int32_t*)(base + T.nbr);
  int32_t* count = (int32_t*)(base + T.count);
  uint32_t* occ = (uint32_t*)(base + T.occ);
  uint32_t* emask = (uint32_t*)(base + T.emask);
  const int threads = 256;
  {
    const int64_t nperm = (int64_t)L.batch * T.nc, ncount = (int64_t)L.batch * nblk;
    const int64_t cnt = nperm > ncount ? nperm : ncount;
    hipLaunchKernelGGL(k_clear, dim3((unsigned)((cnt + threads - 1) / threads)), dim3(threads), 0, s, perm, nperm,
                       count, ncount);
  }
  dim3 tok_grid((unsigned)((L.nmax + threads - 1) / threads), (unsigned)L.batch);
  hipLaunchKernelGGL(k_assign, tok_grid, dim3(threads), 0, s, coords_dev, voff, geom, token_block, canon, perm, count,
                     T.nc, nblk, b);
  hipLaunchKernelGGL(k_dups, tok_grid, dim3(threads), 0, s, canon, voff, perm, geom, T.nc);
  {
    const int32_t words = T.occ_words > T.mask_words ? T.occ_words : T.mask_words;
    dim3 g((unsigned)((words + threads - 1) / threads), (unsigned)L.batch);
    hipLaunchKernelGGL(k_finish, g, dim3(threads), 0, s, perm, occ, count, emask, T.nc, T.occ_words, nblk,
                       T.mask_words);
  }
  {
    const int64_t cnt = (int64_t)nblk * slots;
    dim3 g((unsigned)((cnt + threads - 1) / threads), (unsigned)L.batch);
    hipLaunchKernelGGL(k_nbr, g, dim3(threads), 0, s, geom, nbr, nblk, local_radius, b);
  }
  st = check_launch("build_index");
  if (st != PACK3D_OK) {
    hipStreamSynchronize(s);
    return fail(st);
  }
  st = read_geom(host_geom, geom, L.batch, s);
  if (st != PACK3D_OK) return fail(st);
  int64_t present = 0;
  for (int32_t v = 0; v < L.batch; ++v) {
    const int32_t* g = host_geom + v * G_FIELDS;
    if (g[G_STATUS] != GS_OK) return fail(geometry_error(g, v, b, cap));
    present += g[G_NTOK];
  }
  pack3d_index* ix = (pack3d_index*)std::malloc(sizeof(pack3d_index));
  if (!ix) return fail(set_error(PACK3D_E_INVALID, "build_index: host allocation failed"));
  ix->batch = L.batch; ix->tokens = L.nmax; ix->nblk = nblk; ix->bvol = bvol; ix->slots = slots;
  ix->radius = local_radius;
  ix->ragged = ragged;
  ix->total = L.total;
  ix->holes = present != (int64_t)L.batch * T.nc ? 1 : 0;
  for (int a = 0; a < 3; ++a) {
    ix->block[a] = block_shape[a];
    int32_t m = 0;
    for (int32_t v = 0; v < L.batch; ++v) m = host_geom[v * G_FIELDS + G_EZ + a] > m ? host_geom[v * G_FIELDS + G_EZ + a] : m;
    ix->extent_max[a] = m;
  }
  ix->geom = geom; ix->voff = voff; ix->token_block = token_block; ix->canon = canon; ix->perm = perm; ix->nbr = nbr;
  ix->count = count; ix->occ = occ; ix->emask = emask; ix->occ_words = T.occ_words;
  ix->host_geom = host_geom;
  *out = ix;
  return PACK3D_OK;
}

extern "C" pack3d_status pack3d_index_tables(const pack3d_index* ix, pack3d_tables* out) {
  if (!ix || !out) return set_error(PACK3D_E_INVALID, "index_tables: null pointer argument");
  out->token_block = ix->token_block; out->canon = ix->canon; out->perm = ix->perm;
  out->nbr = ix->nbr; out->geom = ix->geom;
  out->batch = ix->batch; out->tokens = ix->tokens; out->nblk = ix->nblk; out->block_tokens = ix->bvol;
  out->slots = ix->slots; out->radius = ix->radius;
  for (int a = 0; a < 3; ++a) { out->block_shape[a] = ix->block[a]; out->extent_max[a] = ix->extent_max[a]; }
  out->block_count = ix->count; out->volume_offsets = ix->voff; out->total_tokens = ix->total;
  out->ragged = ix->ragged; out->holes = ix->holes;
  return PACK3D_OK;
}

extern "C" pack3d_status pack3d_index_geometry(const pack3d_index* ix, int32_t volume, int32_t out6[6]) {
  if (!ix || !out6) return set_error(PACK3D_E_INVALID, "index_geometry: null pointer argument");
  if (volume < 0 || volume >= ix->batch) return set_error(PACK3D_E_INVALID, "index_geometry: volume out of range");
  for (int f = 0; f < 6; ++f) out6[f] = ix->host_geom[volume * G_FIELDS + f];
  return PACK3D_OK;
}

extern "C" void pack3d_index_free(pack3d_index* ix) {
  if (!ix) return;
  std::free(ix->host_geom);
  std::free(ix);
}
