// Workspace layout and launch parameters shared by the API and the kernels.
#pragma once

#include "common.h"

namespace pack3d {

constexpr int kMaxSlots = 343;        // (2r+1)^3 with r <= 3 in the attention kernels
constexpr int kMaxBlocks = 16384;     // blocks per volume (summary mask in LDS)
constexpr int kMaxBlockTokens = 1024; // tokens per block
constexpr int kTile = 64;             // query rows / key rows per tile

inline int padded_head_dim(int d) { return (d + 31) / 32 * 32; }

struct Dims {
  // NC: canonical rows per volume (nblk * bvol); Nmax: tokens of the largest volume (the
  // lse stride); holes: some canonical slot is empty
  int B, NC, Nmax, H, D, Dp, nblk, nblkp, bvol, slots, emax, holes;
  // rotation: `groups` contiguous head-dim groups of width gw, `half` = gw / 2 pairs
  // (k, k + half) each, table of `trows` angle rows (positions) x half
  int pos_mode, groups, gw, half, trows;
  size_t esize;  // bytes per element of the activation dtype
  // elements between consecutive tokens of the q, k, v inputs and of the dq, dk, dv
  // outputs: H * D for separate [T, H, D] tensors, 3 * H * D inside one [T, 3, H, D] buffer
  int64_t in_stride, grad_stride;
};

inline Dims make_dims(const pack3d_index* ix, const pack3d_attn* at) {
  Dims d;
  d.B = ix->batch; d.NC = ix->nblk * ix->bvol; d.Nmax = ix->tokens; d.H = at->heads; d.D = at->head_dim;
  d.holes = ix->holes;
  d.Dp = padded_head_dim(at->head_dim);
  d.nblk = ix->nblk; d.nblkp = (ix->nblk + kTile - 1) / kTile * kTile;
  d.bvol = ix->bvol; d.slots = ix->slots;
  d.emax = ix->extent_max[0];
  if (ix->extent_max[1] > d.emax) d.emax = ix->extent_max[1];
  if (ix->extent_max[2] > d.emax) d.emax = ix->extent_max[2];
  d.pos_mode = at->position_mode;
  d.groups = d.pos_mode == PACK3D_POS_AXIAL ? 3 : 1;
  d.gw = d.D / d.groups;
  d.half = d.gw / 2;
  d.trows = d.pos_mode == PACK3D_POS_AXIAL ? d.emax : (d.pos_mode == PACK3D_POS_PACKED_1D ? d.Nmax : 1);
  d.esize = at->dtype == PACK3D_BF16 ? 2 : 4;
  d.in_stride = d.grad_stride = (int64_t)d.H * d.D;
  return d;
}

// Query chunks of the summary-major backward: enough workgroups to fill the chip.
inline int summary_chunks(const Dims& d) {
  const int base = (d.nblkp / kTile) * d.H * d.B;
  int qc = 2048 / (base > 0 ? base : 1);
  if (qc < 1) qc = 1;
  if (qc > d.nblk) qc = d.nblk;
  return qc;
}

struct Workspace {
  // forward intermediates (canonical order, row-major)
  size_t rope, qrot, krot, vr, kbar, vbar, fwd_total;
  // backward extras
  size_t doc, lsec, delta, dkbar, dvbar, part_k, part_v, bwd_total;
};

inline Workspace workspace_layout(const Dims& d) {
  Workspace w;
  const size_t bh = (size_t)d.B * d.H;
  const size_t act = bh * d.NC * d.Dp * d.esize;
  const size_t summ = bh * d.nblkp * d.Dp * d.esize;
  const size_t summ32 = bh * d.nblkp * d.Dp * sizeof(float);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.rope = take(sizeof(float) * 2 * (size_t)d.trows * d.half);
  w.qrot = take(act);
  w.krot = take(act);
  w.vr = take(act);
  w.kbar = take(summ);
  w.vbar = take(summ);
  w.fwd_total = off;
  w.doc = take(act);
  w.lsec = take(sizeof(float) * bh * d.NC);
  w.delta = take(sizeof(float) * bh * d.NC);
  w.dkbar = take(summ32);
  w.dvbar = take(summ32);
  w.part_k = take(summ32 * summary_chunks(d));
  w.part_v = take(summ32 * summary_chunks(d));
  w.bwd_total = off;
  return w;
}

// Row of the rotation table for group g of the token at packed position src (its
// coordinates at coords[0..2]): axial mode: the origin-relative coordinate on axis g,
// clamped to the table (in range whenever the coordinates match the index); packed 1D:
// the packed position; no rotation: row 0, whose angle is 0.
__device__ inline int rope_row(int mode, int g, int src, const int32_t* coords, const int32_t* geom, int trows) {
  if (mode == PACK3D_POS_AXIAL) {
    const int r = coords[g] - geom[G_OZ + g];
    return r < 0 ? 0 : (r >= trows ? trows - 1 : r);
  }
  if (mode == PACK3D_POS_PACKED_1D) return src;
  return 0;
}

// Launchers (defined in the kernel sources).
pack3d_status launch_rope_pool(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                               const void* q, const void* k, const void* v, const int32_t* coords,
                               char* ws, const Workspace& w, const char* name, hipStream_t s);
pack3d_status launch_attn_bwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at, const int32_t* coords,
                              const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              char* ws, const Workspace& w, hipStream_t s);
pack3d_status launch_attn_fwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                              const char* ws, const Workspace& w, void* out, float* lse, hipStream_t s);

}  // namespace pack3d
