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
  int B, N, H, D, Dp, nblk, nblkp, bvol, slots, emax, half;
  size_t esize;  // bytes per element of the activation dtype
};

inline Dims make_dims(const pack3d_index* ix, const pack3d_attn* at) {
  Dims d;
  d.B = ix->batch; d.N = ix->tokens; d.H = at->heads; d.D = at->head_dim;
  d.Dp = padded_head_dim(at->head_dim);
  d.nblk = ix->nblk; d.nblkp = (ix->nblk + kTile - 1) / kTile * kTile;
  d.bvol = ix->bvol; d.slots = ix->slots;
  d.emax = ix->extent_max[0];
  if (ix->extent_max[1] > d.emax) d.emax = ix->extent_max[1];
  if (ix->extent_max[2] > d.emax) d.emax = ix->extent_max[2];
  d.half = at->head_dim / 6;
  d.esize = at->dtype == PACK3D_BF16 ? 2 : 4;
  return d;
}

struct Workspace {
  // forward intermediates
  size_t rope, qrot, krot, vt, kbar, vbart, fwd_total;
  // backward extras
  size_t doc, delta, dkbar, dvbar, bwd_total;
};

inline Workspace workspace_layout(const Dims& d) {
  Workspace w;
  const size_t bh = (size_t)d.B * d.H;
  const size_t act = bh * d.N * d.Dp * d.esize;
  size_t off = 0;
  w.rope = off;  off = align_up(off + sizeof(float) * 2 * (size_t)d.emax * d.half, 256);
  w.qrot = off;  off = align_up(off + act, 256);
  w.krot = off;  off = align_up(off + act, 256);
  w.vt = off;    off = align_up(off + act, 256);
  w.kbar = off;  off = align_up(off + bh * d.nblkp * d.Dp * d.esize, 256);
  w.vbart = off; off = align_up(off + bh * d.nblkp * d.Dp * d.esize, 256);
  w.fwd_total = off;
  w.doc = off;   off = align_up(off + act, 256);
  w.delta = off; off = align_up(off + sizeof(float) * bh * d.N, 256);
  w.dkbar = off; off = align_up(off + sizeof(float) * bh * d.nblkp * d.Dp, 256);
  w.dvbar = off; off = align_up(off + sizeof(float) * bh * d.nblkp * d.Dp, 256);
  w.bwd_total = off;
  return w;
}

// Launchers (defined in the kernel sources).
pack3d_status launch_rope_pool(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                               const void* q, const void* k, const void* v, const int32_t* coords,
                               char* ws, const Workspace& w, hipStream_t s);
pack3d_status launch_attn_fwd(const Dims& d, const pack3d_index* ix, const pack3d_attn* at,
                              const char* ws, const Workspace& w, void* out, float* lse, hipStream_t s);

}  // namespace pack3d
