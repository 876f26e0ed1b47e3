// K0: index builder -- block membership, canonical order and neighbour table of
// each packed volume, derived from the tokens' true (z, y, x) grid coordinates.
//
// "Geometry Matters in Packed 3D Attention" (abstract): the operator separates the
// memory layout from the attention geometry, so every table here is a function of
// the coordinates alone; the packing order only decides where each token's entry
// is stored.  Readings: the block lattice is anchored at each volume's componentwise
// minimum coordinate; only full grids whose extents divide by the block are
// accepted; the local set is block-granular (Chebyshev radius r in block units).
//
// Kernels (all integer, exact):
//   init      geom <- sentinels, perm <- INT_MAX
//   extents   per-volume componentwise min / max (atomicMin / atomicMax)
//   check     per-volume extent product and divisibility -> status
//   assign    per token: block id, canonical slot, atomicMin(perm[slot], token)
//   dups      per token: perm[slot] != token -> duplicate; lowest such token kept
//   nbr       per (volume, block, slot): neighbour id or -1
#include <climits>
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace pack3d {
namespace {

__global__ void k_init(int32_t* geom, int32_t* perm, int32_t batch, int64_t total) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)batch * G_FIELDS) {
    int f = (int)(i % G_FIELDS);
    int32_t v = 0;
    if (f <= G_OX) v = INT_MAX;                      // running minimum
    else if (f <= G_EX) v = INT_MIN;                 // running maximum (turned into extent later)
    else if (f == G_STATUS) v = GS_OK;
    else v = INT_MAX;                                // offending token (minimum)
    geom[i] = v;
  }
  if (i < total) perm[i] = INT_MAX;
}

// One thread per token; wave-level reduction before the atomics.
__global__ void k_extents(const int32_t* __restrict__ coords, int32_t* geom, int32_t n) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  int32_t mn[3] = {INT_MAX, INT_MAX, INT_MAX}, mx[3] = {INT_MIN, INT_MIN, INT_MIN};
  if (i < n) {
    const int32_t* c = coords + ((int64_t)vol * n + i) * 3;
    for (int a = 0; a < 3; ++a) mn[a] = mx[a] = c[a];
  }
  for (int a = 0; a < 3; ++a) {
    for (int off = 32; off > 0; off >>= 1) {
      mn[a] = min(mn[a], __shfl_xor(mn[a], off));
      mx[a] = max(mx[a], __shfl_xor(mx[a], off));
    }
  }
  if ((threadIdx.x & 63) == 0) {
    int32_t* g = geom + vol * G_FIELDS;
    for (int a = 0; a < 3; ++a) {
      atomicMin(g + G_OZ + a, mn[a]);
      atomicMax(g + G_EZ + a, mx[a]);
    }
  }
}

// One thread per volume: max -> extent, then validate the grid.
__global__ void k_check(int32_t* geom, int32_t batch, int32_t n, int32_t bz, int32_t by, int32_t bx) {
  const int32_t vol = blockIdx.x * blockDim.x + threadIdx.x;
  if (vol >= batch) return;
  int32_t* g = geom + vol * G_FIELDS;
  int64_t e[3];
  for (int a = 0; a < 3; ++a) e[a] = (int64_t)g[G_EZ + a] - (int64_t)g[G_OZ + a] + 1;
  int status = GS_OK;
  // product of extents == n, computed without overflow (each extent <= n first)
  if (e[0] > n || e[1] > n || e[2] > n) status = GS_GRID;
  else if (e[0] * e[1] > n || e[0] * e[1] * e[2] != n) status = GS_GRID;
  else if (e[0] % bz || e[1] % by || e[2] % bx) status = GS_DIVISIBLE;
  for (int a = 0; a < 3; ++a) g[G_EZ + a] = (int32_t)(e[a] > INT_MAX ? INT_MAX : e[a]);
  g[G_STATUS] = status;
}

struct BlockShape { int32_t bz, by, bx, bvol; };

__device__ inline bool token_slot(const int32_t* c, const int32_t* g, BlockShape b,
                                  int32_t& blk, int32_t& slot) {
  int32_t rz = c[0] - g[G_OZ], ry = c[1] - g[G_OY], rx = c[2] - g[G_OX];
  int32_t nby = g[G_EY] / b.by, nbx = g[G_EX] / b.bx;
  int32_t qz = rz / b.bz, qy = ry / b.by, qx = rx / b.bx;
  blk = (qz * nby + qy) * nbx + qx;
  int32_t w = ((rz - qz * b.bz) * b.by + (ry - qy * b.by)) * b.bx + (rx - qx * b.bx);
  slot = blk * b.bvol + w;
  return true;
}

__global__ void k_assign(const int32_t* __restrict__ coords, const int32_t* __restrict__ geom,
                         int32_t* token_block, int32_t* canon, int32_t* perm, int32_t n, BlockShape b) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t* g = geom + vol * G_FIELDS;
  const int64_t t = (int64_t)vol * n + i;
  if (g[G_STATUS] != GS_OK) {
    token_block[t] = -1;
    canon[t] = -1;
    return;
  }
  int32_t blk, slot;
  token_slot(coords + t * 3, g, b, blk, slot);   // in range: the grid check passed
  token_block[t] = blk;
  canon[t] = slot;
  atomicMin(perm + (int64_t)vol * n + slot, i);
}

__global__ void k_dups(const int32_t* __restrict__ canon, const int32_t* __restrict__ perm, int32_t* geom, int32_t n) {
  const int32_t vol = blockIdx.y;
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int32_t* g = geom + vol * G_FIELDS;
  if (g[G_STATUS] != GS_OK && g[G_STATUS] != GS_DUPLICATE) return;
  const int32_t s = canon[(int64_t)vol * n + i];
  if (s < 0) return;
  if (perm[(int64_t)vol * n + s] != i) {
    atomicMin(g + G_TOKEN, i);
    g[G_STATUS] = GS_DUPLICATE;  // every writer stores the same value
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
  if (g[G_STATUS] != GS_OK) { out[i] = -1; return; }
  const int32_t blk = (int32_t)(i / slots), s = (int32_t)(i % slots);
  const int32_t nbz = g[G_EZ] / b.bz, nby = g[G_EY] / b.by, nbx = g[G_EX] / b.bx;
  const int32_t z = blk / (nby * nbx), y = (blk / nbx) % nby, x = blk % nbx;
  const int32_t dz = s / (span * span) - radius, dy = (s / span) % span - radius, dx = s % span - radius;
  const int32_t zz = z + dz, yy = y + dy, xx = x + dx;
  const bool in = zz >= 0 && zz < nbz && yy >= 0 && yy < nby && xx >= 0 && xx < nbx;
  out[i] = in ? (zz * nby + yy) * nbx + xx : -1;
}

struct TableLayout {
  size_t geom, token_block, canon, perm, nbr, total;
};

TableLayout table_layout(int32_t batch, int32_t n, int32_t nblk, int32_t slots) {
  TableLayout t;
  size_t off = 0;
  t.geom = off;        off = align_up(off + sizeof(int32_t) * batch * G_FIELDS, 256);
  t.token_block = off; off = align_up(off + sizeof(int32_t) * (size_t)batch * n, 256);
  t.canon = off;       off = align_up(off + sizeof(int32_t) * (size_t)batch * n, 256);
  t.perm = off;        off = align_up(off + sizeof(int32_t) * (size_t)batch * n, 256);
  t.nbr = off;         off = align_up(off + sizeof(int32_t) * (size_t)batch * nblk * slots, 256);
  t.total = off;
  return t;
}

bool valid_args(const pack3d_packing* p, const int32_t* block, int32_t r) {
  if (!p || !block) return false;
  if (p->batch < 1 || p->tokens_per_volume < 1) return false;
  if (block[0] < 1 || block[1] < 1 || block[2] < 1) return false;
  if (r < 0) return false;
  return true;
}

}  // namespace
}  // namespace pack3d

using namespace pack3d;

extern "C" size_t pack3d_index_bytes(const pack3d_packing* packing, const int32_t block_shape[3],
                                     int32_t local_radius) {
  if (!valid_args(packing, block_shape, local_radius) || local_radius > 7) return 0;
  const int64_t bvol = (int64_t)block_shape[0] * block_shape[1] * block_shape[2];
  if (bvol > packing->tokens_per_volume || packing->tokens_per_volume % bvol) return 0;
  const int32_t span = 2 * local_radius + 1;
  return table_layout(packing->batch, packing->tokens_per_volume,
                      (int32_t)(packing->tokens_per_volume / bvol), span * span * span).total;
}

extern "C" pack3d_status pack3d_build_index(const int32_t* coords_dev, const pack3d_packing* packing,
                                            const int32_t block_shape[3], int32_t local_radius,
                                            void* tables_dev, size_t tables_bytes, void* stream,
                                            pack3d_index** out) {
  if (out) *out = nullptr;
  if (!coords_dev || !tables_dev || !out)
    return set_error(PACK3D_E_INVALID, "build_index: null pointer argument");
  if (!valid_args(packing, block_shape, local_radius))
    return set_error(PACK3D_E_INVALID, "build_index: batch and tokens must be >= 1, block extents >= 1, radius >= 0");
  if (local_radius > 7)
    return set_error(PACK3D_E_UNSUPPORTED, "build_index: local_radius %d > 7 is not supported", local_radius);
  const int32_t batch = packing->batch, n = packing->tokens_per_volume;
  const int64_t bvol64 = (int64_t)block_shape[0] * block_shape[1] * block_shape[2];
  if (bvol64 > n || n % bvol64)
    return set_error(PACK3D_E_COORDS, "build_index: %d tokens per volume cannot tile into %lld-token blocks",
                     n, (long long)bvol64);
  if (bvol64 % 8)
    return set_error(PACK3D_E_UNSUPPORTED, "build_index: block volume %lld is not a multiple of 8",
                     (long long)bvol64);
  if (bvol64 > 64 && bvol64 % 64)
    return set_error(PACK3D_E_UNSUPPORTED,
                     "build_index: block volume %lld above 64 must be a multiple of 64", (long long)bvol64);
  if ((int64_t)batch * n > INT32_MAX)
    return set_error(PACK3D_E_UNSUPPORTED, "build_index: batch * tokens exceeds 2^31 - 1");
  const int32_t bvol = (int32_t)bvol64, nblk = n / bvol;
  const int32_t span = 2 * local_radius + 1, slots = span * span * span;
  const TableLayout L = table_layout(batch, n, nblk, slots);
  if (tables_bytes < L.total)
    return set_error(PACK3D_E_WORKSPACE, "build_index: tables buffer %zu bytes < %zu needed", tables_bytes, L.total);

  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)tables_dev;
  int32_t* geom = (int32_t*)(base + L.geom);
  int32_t* token_block = (int32_t*)(base + L.token_block);
  int32_t* canon = (int32_t*)(base + L.canon);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* nbr = (int32_t*)(base + L.nbr);
  BlockShape b{block_shape[0], block_shape[1], block_shape[2], bvol};
  const int64_t total = (int64_t)batch * n;
  const int threads = 256;
  {
    int64_t cnt = total > (int64_t)batch * G_FIELDS ? total : (int64_t)batch * G_FIELDS;
    hipLaunchKernelGGL(k_init, dim3((unsigned)((cnt + threads - 1) / threads)), dim3(threads), 0, s,
                       geom, perm, batch, total);
  }
  dim3 tok_grid((unsigned)((n + threads - 1) / threads), (unsigned)batch);
  hipLaunchKernelGGL(k_extents, tok_grid, dim3(threads), 0, s, coords_dev, geom, n);
  hipLaunchKernelGGL(k_check, dim3((batch + 63) / 64), dim3(64), 0, s, geom, batch, n, b.bz, b.by, b.bx);
  hipLaunchKernelGGL(k_assign, tok_grid, dim3(threads), 0, s, coords_dev, geom, token_block, canon, perm, n, b);
  hipLaunchKernelGGL(k_dups, tok_grid, dim3(threads), 0, s, canon, perm, geom, n);
  {
    int64_t cnt = (int64_t)nblk * slots;
    dim3 g((unsigned)((cnt + threads - 1) / threads), (unsigned)batch);
    hipLaunchKernelGGL(k_nbr, g, dim3(threads), 0, s, geom, nbr, nblk, local_radius, b);
  }
  pack3d_status st = check_launch("build_index");
  if (st != PACK3D_OK) return st;

  int32_t* host_geom = (int32_t*)std::malloc(sizeof(int32_t) * batch * G_FIELDS);
  if (!host_geom) return set_error(PACK3D_E_INVALID, "build_index: host allocation failed");
  hipError_t e = hipMemcpyAsync(host_geom, geom, sizeof(int32_t) * batch * G_FIELDS, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    std::free(host_geom);
    return set_error(PACK3D_E_HIP, "build_index: %s", hipGetErrorString(e));
  }
  for (int32_t v = 0; v < batch; ++v) {
    const int32_t* g = host_geom + v * G_FIELDS;
    if (g[G_STATUS] != GS_OK) {
      pack3d_status r;
      if (g[G_STATUS] == GS_GRID)
        r = set_error(PACK3D_E_COORDS, "build_index: volume %d: coordinates do not fill their bounding box "
                      "(extent %d x %d x %d for %d tokens)", v, g[G_EZ], g[G_EY], g[G_EX], n);
      else if (g[G_STATUS] == GS_DIVISIBLE)
        r = set_error(PACK3D_E_COORDS, "build_index: volume %d: extent %d x %d x %d not divisible by block "
                      "%d x %d x %d", v, g[G_EZ], g[G_EY], g[G_EX], b.bz, b.by, b.bx);
      else
        r = set_error(PACK3D_E_COORDS, "build_index: volume %d: duplicate point at packed index %d", v, g[G_TOKEN]);
      std::free(host_geom);
      return r;
    }
  }
  pack3d_index* ix = (pack3d_index*)std::malloc(sizeof(pack3d_index));
  if (!ix) {
    std::free(host_geom);
    return set_error(PACK3D_E_INVALID, "build_index: host allocation failed");
  }
  ix->batch = batch; ix->tokens = n; ix->nblk = nblk; ix->bvol = bvol; ix->slots = slots;
  ix->radius = local_radius;
  for (int a = 0; a < 3; ++a) {
    ix->block[a] = block_shape[a];
    int32_t m = 0;
    for (int32_t v = 0; v < batch; ++v) m = host_geom[v * G_FIELDS + G_EZ + a] > m ? host_geom[v * G_FIELDS + G_EZ + a] : m;
    ix->extent_max[a] = m;
  }
  ix->geom = geom; ix->token_block = token_block; ix->canon = canon; ix->perm = perm; ix->nbr = nbr;
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
