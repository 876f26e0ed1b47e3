// C ABI entry points of libpack3d: argument checks, workspace layout, dispatch.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "layout.h"

// Device scratch of pack3d_forward_noalloc: the forward's workspace for callers that cannot
// allocate.  Every GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory: kernels get the
// address hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static constexpr size_t kNoAllocBytes = PACK3D_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kNoAllocBytes];

namespace pack3d {

static thread_local char g_msg[512] = "";

pack3d_status set_error(pack3d_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

pack3d_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PACK3D_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return PACK3D_OK;
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

pack3d_status check_attn(const pack3d_index* ix, const pack3d_attn* at, const char* who) {
  if (!ix || !at) return set_error(PACK3D_E_INVALID, "%s: null index or attention parameters", who);
  if (at->dtype != PACK3D_F32 && at->dtype != PACK3D_BF16)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: dtype %d is not supported", who, at->dtype);
  if (at->heads < 1) return set_error(PACK3D_E_INVALID, "%s: heads must be >= 1", who);
  if (at->head_dim < 6 || at->head_dim % 6 || at->head_dim > 128)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: head_dim %d must be a multiple of 6 in [6, 128]", who, at->head_dim);
  if (at->position_mode != PACK3D_POS_AXIAL && at->position_mode != PACK3D_POS_PACKED_1D &&
      at->position_mode != PACK3D_POS_NONE)
    return set_error(PACK3D_E_INVALID, "%s: position_mode %d is not one of 0, 1, 2", who, at->position_mode);
  if (!(at->rope_base > 0.0f) || !std::isfinite(at->rope_base))
    return set_error(PACK3D_E_INVALID, "%s: rope_base must be positive and finite", who);
  if (!std::isfinite(at->softmax_scale))
    return set_error(PACK3D_E_INVALID, "%s: softmax_scale must be finite", who);
  if (ix->slots > kMaxSlots)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: local radius %d > 3 is not supported by the attention kernels",
                     who, ix->radius);
  if (ix->nblk > kMaxBlocks)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: %d blocks per volume > %d", who, ix->nblk, kMaxBlocks);
  if (ix->bvol > kMaxBlockTokens)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: %d tokens per block > %d", who, ix->bvol, kMaxBlockTokens);
  if ((int64_t)ix->batch * at->heads * ix->nblk * ix->bvol * padded_head_dim(at->head_dim) > ((int64_t)1 << 40))
    return set_error(PACK3D_E_UNSUPPORTED, "%s: problem too large", who);
  return PACK3D_OK;
}

}  // namespace
}  // namespace pack3d

using namespace pack3d;

extern "C" const char* pack3d_last_error(void) { return g_msg; }

extern "C" int32_t pack3d_version(void) { return 104; }

extern "C" size_t pack3d_workspace_bytes(const pack3d_index* ix, const pack3d_attn* at, int for_backward) {
  if (check_attn(ix, at, "workspace_bytes") != PACK3D_OK) return 0;
  Workspace w = workspace_layout(make_dims(ix, at));
  return for_backward ? w.bwd_total : w.fwd_total;
}

extern "C" pack3d_status pack3d_workspace_views(const pack3d_index* ix, const pack3d_attn* at, pack3d_views* out) {
  pack3d_status st = check_attn(ix, at, "workspace_views");
  if (st != PACK3D_OK) return st;
  if (!out) return set_error(PACK3D_E_INVALID, "workspace_views: null output");
  Dims d = make_dims(ix, at);
  Workspace w = workspace_layout(d);
  out->rope_table = w.rope; out->qrot = w.qrot; out->krot = w.krot; out->vrow = w.vr;
  out->kbar = w.kbar; out->vbar = w.vbar;
  out->head_dim_padded = d.Dp; out->nblk_padded = d.nblkp; out->extent_table = d.trows;
  return PACK3D_OK;
}

namespace {

// q, k, v (and dq, dk, dv) are tokens of `in_stride` (`grad_stride`) elements apart.
pack3d_status run_forward(const pack3d_index* ix, const pack3d_attn* at, const void* q, const void* k,
                          const void* v, const int32_t* coords, void* out, float* lse, void* ws, size_t ws_bytes,
                          int64_t in_stride, void* stream, const char* who) {
  pack3d_status st = check_attn(ix, at, who);
  if (st != PACK3D_OK) return st;
  if (!q || !k || !v || !coords || !out || !lse || !ws)
    return set_error(PACK3D_E_INVALID, "%s: null pointer argument", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws))
    return set_error(PACK3D_E_INVALID, "%s: q, k, v, out and workspace must be 16-byte aligned", who);
  Dims d = make_dims(ix, at);
  d.in_stride = in_stride;
  Workspace w = workspace_layout(d);
  if (ws_bytes < w.fwd_total)
    return set_error(PACK3D_E_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, w.fwd_total);
  hipStream_t s = (hipStream_t)stream;
  st = launch_rope_pool(d, ix, at, q, k, v, coords, (char*)ws, w, "rope_pool", s);
  if (st != PACK3D_OK) return st;
  return launch_attn_fwd(d, ix, at, (const char*)ws, w, out, lse, s);
}

pack3d_status run_backward(const pack3d_index* ix, const pack3d_attn* at, const void* q, const void* k,
                           const void* v, const int32_t* coords, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                           int32_t reuse_forward, int64_t in_stride, int64_t grad_stride, void* stream,
                           const char* who) {
  pack3d_status st = check_attn(ix, at, who);
  if (st != PACK3D_OK) return st;
  if (!q || !k || !v || !coords || !out || !lse || !dout || !dq || !dk || !dv || !ws)
    return set_error(PACK3D_E_INVALID, "%s: null pointer argument", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(ws) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return set_error(PACK3D_E_INVALID, "%s: q, k, v, out, dout, dq, dk, dv and workspace must be 16-byte aligned",
                     who);
  Dims d = make_dims(ix, at);
  d.in_stride = in_stride;
  d.grad_stride = grad_stride;
  Workspace w = workspace_layout(d);
  if (ws_bytes < w.bwd_total)
    return set_error(PACK3D_E_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, w.bwd_total);
  if (reuse_forward != 0 && reuse_forward != 1)
    return set_error(PACK3D_E_INVALID, "%s: reuse_forward must be 0 or 1", who);
  hipStream_t s = (hipStream_t)stream;
  if (!reuse_forward) {
    // recompute the rotated and pooled operands into the forward part of the workspace
    st = launch_rope_pool(d, ix, at, q, k, v, coords, (char*)ws, w, "rope_pool_bwd", s);
    if (st != PACK3D_OK) return st;
  }
  return launch_attn_bwd(d, ix, at, coords, out, lse, dout, dq, dk, dv, (char*)ws, w, s);
}

// Device address of `scratch` on the current device, taken once per device with that
// device current and kept; later calls reuse it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

pack3d_status noalloc_scratch(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(PACK3D_E_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: device %d is beyond the %d devices supported", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(PACK3D_E_HIP, "%s: hipGetSymbolAddress of the scratch buffer on device %d: %s", who, dev,
                       hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return PACK3D_OK;
}

// The fused [T, 3, H, D] layout needs every head block (H * D elements) to start on a
// 16-byte boundary.
pack3d_status check_fused(const pack3d_attn* at, const char* who) {
  if (!at) return set_error(PACK3D_E_INVALID, "%s: null attention parameters", who);
  const size_t es = at->dtype == PACK3D_BF16 ? 2 : 4;
  if (((size_t)at->heads * at->head_dim * es) % 16)
    return set_error(PACK3D_E_UNSUPPORTED, "%s: heads * head_dim * element size must be a multiple of 16 bytes",
                     who);
  return PACK3D_OK;
}

}  // namespace

extern "C" pack3d_status pack3d_forward(const pack3d_index* ix, const pack3d_attn* at, const void* q,
                                        const void* k, const void* v, const int32_t* coords, void* out,
                                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  const int64_t hd = at ? (int64_t)at->heads * at->head_dim : 0;
  return run_forward(ix, at, q, k, v, coords, out, lse, ws, ws_bytes, hd, stream, "forward");
}

extern "C" pack3d_status pack3d_forward_noalloc(const pack3d_index* ix, const pack3d_attn* at, const void* q,
                                                const void* k, const void* v, const int32_t* coords, void* out,
                                                float* lse, void* stream) {
  const char* who = "forward_noalloc";
  pack3d_status st = check_attn(ix, at, who);
  if (st != PACK3D_OK) return st;
  const size_t need = workspace_layout(make_dims(ix, at)).fwd_total;
  if (need > kNoAllocBytes)
    return set_error(PACK3D_E_WORKSPACE,
                     "%s: this forward needs %zu bytes of workspace, more than the %zu bytes of the fixed device "
                     "scratch buffer; call pack3d_forward with a caller workspace instead",
                     who, need, kNoAllocBytes);
  void* ws = nullptr;
  st = noalloc_scratch(&ws, who);
  if (st != PACK3D_OK) return st;
  ProfileOff quiet;  // kernel timing would create events
  const int64_t hd = (int64_t)at->heads * at->head_dim;
  return run_forward(ix, at, q, k, v, coords, out, lse, ws, kNoAllocBytes, hd, stream, who);
}

extern "C" pack3d_status pack3d_backward(const pack3d_index* ix, const pack3d_attn* at, const void* q,
                                         const void* k, const void* v, const int32_t* coords,
                                         const void* out, const float* lse, const void* dout, void* dq,
                                         void* dk, void* dv, void* ws, size_t ws_bytes, int32_t reuse_forward,
                                         void* stream) {
  const int64_t hd = at ? (int64_t)at->heads * at->head_dim : 0;
  return run_backward(ix, at, q, k, v, coords, out, lse, dout, dq, dk, dv, ws, ws_bytes, reuse_forward, hd, hd,
                      stream, "backward");
}

extern "C" pack3d_status pack3d_forward_qkv(const pack3d_index* ix, const pack3d_attn* at, const void* qkv,
                                            const int32_t* coords, void* out, float* lse, void* ws,
                                            size_t ws_bytes, void* stream) {
  pack3d_status st = check_fused(at, "forward_qkv");
  if (st != PACK3D_OK) return st;
  if (!qkv) return set_error(PACK3D_E_INVALID, "forward_qkv: null pointer argument");
  const int64_t hd = (int64_t)at->heads * at->head_dim;
  const size_t part = (size_t)hd * (at->dtype == PACK3D_BF16 ? 2 : 4);
  const char* base = (const char*)qkv;
  return run_forward(ix, at, base, base + part, base + 2 * part, coords, out, lse, ws, ws_bytes, 3 * hd, stream,
                     "forward_qkv");
}

extern "C" pack3d_status pack3d_backward_qkv(const pack3d_index* ix, const pack3d_attn* at, const void* qkv,
                                             const int32_t* coords, const void* out, const float* lse,
                                             const void* dout, void* dqkv, void* ws, size_t ws_bytes,
                                             int32_t reuse_forward, void* stream) {
  pack3d_status st = check_fused(at, "backward_qkv");
  if (st != PACK3D_OK) return st;
  if (!qkv || !dqkv) return set_error(PACK3D_E_INVALID, "backward_qkv: null pointer argument");
  if (!aligned16(dqkv)) return set_error(PACK3D_E_INVALID, "backward_qkv: dqkv must be 16-byte aligned");
  const int64_t hd = (int64_t)at->heads * at->head_dim;
  const size_t part = (size_t)hd * (at->dtype == PACK3D_BF16 ? 2 : 4);
  const char* base = (const char*)qkv;
  char* g = (char*)dqkv;
  return run_backward(ix, at, base, base + part, base + 2 * part, coords, out, lse, dout, g, g + part, g + 2 * part,
                      ws, ws_bytes, reuse_forward, 3 * hd, 3 * hd, stream, "backward_qkv");
}
