/*
 * pack3d.h -- C ABI of the PACK3D local-global attention operator for MI355X (gfx950).
 *
 * The operator ("Geometry Matters in Packed 3D Attention", arXiv:2610.38694, abstract):
 * every token of a packed 3D volume attends exactly to the keys of its 3D
 * neighbourhood of blocks, and to one summary per distant contiguous 3D block,
 * under one shared softmax.  Every query-key and query-summary logit is indexed by
 * axial RoPE on the tokens' true (z, y, x) grid coordinates, never their packed
 * position, and the rotation is applied before a block is summarized (a summary is
 * the mean of the block's rotated keys and the mean of its values).
 *
 * Conventions shared by every entry point
 *   - Every pointer named *_dev is device memory owned by the caller; the library
 *     never allocates, frees or retains device memory.  It allocates only the small
 *     host-side index handle (malloc/free).
 *   - q, k, v, out, dout, dq, dk, dv are contiguous [T, H, D] arrays, D innermost,
 *     in packed (caller) order, all of the dtype named in pack3d_attn: volume v owns
 *     tokens off[v] .. off[v+1]-1 (uniform layout: off[v] = v N, i.e. [B, N, H, D]).
 *     lse is fp32 [B, H, Nmax] in packed order inside each volume (Nmax = the largest
 *     volume; entries past a volume's token count are not written).  coords is int32
 *     [T, 3] holding (z, y, x).
 *   - stream is a hipStream_t (NULL = the null stream).  Forward and backward are
 *     asynchronous on it and never synchronize.  pack3d_build_index synchronizes the
 *     stream once (twice for ragged geometry) to read back the geometry check;
 *     pack3d_measure_blocks synchronizes it once.
 *   - On any error nothing is launched (argument errors) and a message is kept in a
 *     thread-local buffer returned by pack3d_last_error().  Launch failures return
 *     PACK3D_E_HIP.
 *   - Functions never throw and are safe to call from several host threads on
 *     different handles; calls sharing a workspace must be serialized by the caller.
 */
#ifndef PACK3D_H
#define PACK3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pack3d_status {
  PACK3D_OK = 0,
  PACK3D_E_INVALID = 1,     /* null pointer, non-positive size, bad radius or block shape */
  PACK3D_E_COORDS = 2,      /* geometry rejected: not a full grid or extents not divisible
                               by the block (without ragged), a duplicate point, an empty
                               volume, more blocks than the tables were sized for */
  PACK3D_E_UNSUPPORTED = 3, /* valid request outside what the kernels implement */
  PACK3D_E_WORKSPACE = 4,   /* caller buffer smaller than the size query returned */
  PACK3D_E_HIP = 5          /* HIP runtime or launch error */
} pack3d_status;

typedef enum pack3d_dtype { PACK3D_F32 = 0, PACK3D_BF16 = 1 } pack3d_dtype;

/* A hint only: results never depend on it (the coordinates alone define geometry). */
typedef enum pack3d_order {
  PACK3D_ORDER_ANY = 0,
  PACK3D_ORDER_RASTER = 1,
  PACK3D_ORDER_MORTON = 2,
  PACK3D_ORDER_BLOCK_CONTIGUOUS = 3,
  PACK3D_ORDER_RANDOM = 4
} pack3d_order;

/* Batch layout and geometry class.
 *   batch:             number of volumes B.
 *   tokens_per_volume: uniform layout (volume_offsets NULL): tokens N of every volume.
 *                      Ignored with volume_offsets.
 *   order_hint:        pack3d_order.
 *   ragged:            0: every volume must be a full grid (N = product of its extents)
 *                      whose extents the block divides (PACK3D_E_COORDS otherwise).
 *                      1: a volume is any set of distinct integer points: partial edge
 *                      blocks and holes ("Geometry Matters in Packed 3D Attention",
 *                      abstract: packed geometric data).  Blocks cover each volume's
 *                      bounding box from its minimum corner (ceil(extent / b) per axis);
 *                      the local set is the tokens present in the blocks within the
 *                      radius; each other occupied block gives one summary, the mean
 *                      over its tokens; an empty block gives none.
 *   volume_offsets:    NULL, or a host array of batch + 1 token offsets (off[0] = 0,
 *                      non-decreasing, every volume non-empty) for volumes of different
 *                      token counts (varlen batch); read during the call only.
 *   max_blocks:        ragged only: blocks per volume the index tables are sized for
 *                      (pack3d_measure_blocks gives the exact need).  Ignored otherwise. */
typedef struct pack3d_packing {
  int32_t batch;
  int32_t tokens_per_volume;
  int32_t order_hint; /* pack3d_order */
  int32_t ragged;
  const int32_t* volume_offsets;
  int32_t max_blocks;
} pack3d_packing;

/* Angle source of the rotation ("Geometry Matters in Packed 3D Attention", abstract: the
 * operator indexes every interaction with axial RoPE on grid coordinates rather than packed
 * positions, and packed-position encodings break under repacking).  Locality and summaries
 * always follow the grid; only the rotation of Q and K changes.
 *   PACK3D_POS_AXIAL:     the method: head dim split into (z, y, x) groups of D/3, pairs
 *                         (k, k + D/6), angle = grid coordinate * base^(-2k/(D/3)).
 *   PACK3D_POS_PACKED_1D: control: standard 1D RoPE on the packed sequence position (the
 *                         token's index in its volume), pairs (k, k + D/2), angle =
 *                         position * base^(-2k/D) ("SpatioTemporal RoPE" section, 1D form).
 *   PACK3D_POS_NONE:      control: no rotation. */
typedef enum pack3d_position_mode {
  PACK3D_POS_AXIAL = 0,
  PACK3D_POS_PACKED_1D = 1,
  PACK3D_POS_NONE = 2
} pack3d_position_mode;

/* Attention parameters.
 *   head_dim: D, split into three axis groups (z, y, x) of D/3 each; D % 6 == 0 and
 *             D <= 128 (inside each group element k pairs with element k + D/6).
 *   rope_base: base of the RoPE frequencies theta_k = base^(-2k/(D/3)) (e.g. 10000).
 *   softmax_scale: <= 0 selects 1/sqrt(D).
 *   with_summaries: 1 = PACK3D (local keys + distant block summaries),
 *                   0 = windowed-only (local keys only; the latency baseline).
 *   position_mode:  pack3d_position_mode (0 = the method). */
typedef struct pack3d_attn {
  int32_t dtype; /* pack3d_dtype */
  int32_t heads;
  int32_t head_dim;
  float rope_base;
  float softmax_scale;
  int32_t with_summaries;
  int32_t position_mode; /* pack3d_position_mode */
} pack3d_attn;

/* Opaque host handle describing one geometry (built once, reused by every call). */
typedef struct pack3d_index pack3d_index;

/* Device views of the index tables (read-only; they live in the caller's tables_dev).
 * nblk is the largest block count of the batch; a volume with fewer blocks has empty
 * ones past its own count.  Local indices count tokens inside a volume.
 *   token_block [T]         block id of each packed token; blocks are numbered in raster
 *                           order over the block grid (z slowest) of its volume
 *   canon       [T]         canonical slot of each packed token: block id * |b| + raster
 *                           offset inside the block
 *   perm        [B, nblk |b|]  local packed index stored at each canonical slot (inverse
 *                           of canon), -1 for an empty slot
 *   nbr         [B, nblk, slots]  block ids of the (2r+1)^3 neighbourhood of each block,
 *                           slots in raster order over (dz, dy, dx) in [-r, r]^3, -1 outside
 *                           the volume's block grid (a whole row of -1 past its blocks)
 *   block_count [B, nblk]   tokens present in each block
 *   volume_offsets [B + 1]  token offset of each volume
 *   geom        [B, 10]     origin (z, y, x) = componentwise minimum coordinate, extent
 *                           (z, y, x), status, offending token, tokens, blocks of the
 *                           volume (device copy)                                       */
typedef struct pack3d_tables {
  const int32_t* token_block;
  const int32_t* canon;
  const int32_t* perm;
  const int32_t* nbr;
  const int32_t* geom;
  int32_t batch, tokens, nblk, block_tokens, slots, radius;
  int32_t block_shape[3];
  int32_t extent_max[3];
  const int32_t* block_count;
  const int32_t* volume_offsets;
  int64_t total_tokens;
  int32_t ragged, holes; /* holes: some canonical slot is empty */
} pack3d_tables;

/* Plumbing (no passage of the pages defines this call): device bytes needed for the
 * index tables of this batch layout, block shape and radius; 0 if the arguments are
 * invalid.  Without ragged the count follows from the
 * token counts (a valid volume has N_v / |b| blocks); with ragged it is sized for
 * packing->max_blocks blocks per volume. */
size_t pack3d_index_bytes(const pack3d_packing* packing, const int32_t block_shape[3],
                          int32_t local_radius);

/* Plumbing for ragged geometry (no passage defines this call; it sizes the tables of the
 * reading of packed geometric data above): the number of blocks per volume (the largest
 * over the batch) that the coordinates need, i.e. the product over the axes of ceil(extent / b), into
 * *max_blocks_out.  scratch_dev: device buffer of at least 64 * batch bytes.  Runs on the
 * stream and synchronizes it once.  PACK3D_E_COORDS for an empty volume. */
pack3d_status pack3d_measure_blocks(const int32_t* coords_dev, const pack3d_packing* packing,
                                    const int32_t block_shape[3], void* scratch_dev,
                                    size_t scratch_bytes, void* stream, int32_t* max_blocks_out);

/* Build the index of a batch of packed volumes ("Geometry Matters in Packed 3D Attention",
 * abstract: the operator separates memory layout from attention geometry, so locality and
 * the contiguous 3D blocks are derived from the tokens' true grid coordinates, never from
 * their packed positions; the tables are therefore the same, up to the packing
 * permutation, under any repacking).
 *   coords_dev [T, 3] int32 (z, y, x) grid coordinates in packed order.
 *   block_shape (bz, by, bx) >= 1 with bz*by*bx a multiple of 8; local_radius r in
 *   block units (0 <= r <= 7): a query's local set is every key whose block is within
 *   Chebyshev distance r of the query's block (truncated at the volume edge); every
 *   other block of the same volume contributes one summary.
 *   tables_dev / tables_bytes: caller device buffer of at least pack3d_index_bytes();
 *   it must outlive the handle.
 * Each volume's block lattice is anchored at its componentwise minimum coordinate.
 * Rejected with PACK3D_E_COORDS (message names the volume and, for a duplicate, the
 * lowest local index whose point already occurs earlier in the volume): without ragged,
 * extents whose product is not N (holes) or that the block does not divide; always,
 * duplicate points; with ragged, more blocks than packing->max_blocks.
 * On success *out receives a handle to release with pack3d_index_free. */
pack3d_status pack3d_build_index(const int32_t* coords_dev, const pack3d_packing* packing,
                                 const int32_t block_shape[3], int32_t local_radius,
                                 void* tables_dev, size_t tables_bytes, void* stream,
                                 pack3d_index** out);

/* Plumbing (no passage defines this call): fill *out with device views of the tables
 * and their sizes. */
pack3d_status pack3d_index_tables(const pack3d_index* index, pack3d_tables* out);

/* Plumbing (no passage defines this call): host copy of one volume's origin and extent: out6 = (oz, oy, ox, ez, ey, ex) (the extent
 * of the coordinates' bounding box). */
pack3d_status pack3d_index_geometry(const pack3d_index* index, int32_t volume, int32_t out6[6]);

/* Plumbing (no passage defines this call): release a handle (NULL is ignored); the caller
 * still owns tables_dev. */
void pack3d_index_free(pack3d_index* index);

/* Plumbing (no passage defines this call): device workspace bytes for pack3d_forward
 * (for_backward = 0) or pack3d_backward (for_backward = 1); 0 if the request is invalid
 * or unsupported. */
size_t pack3d_workspace_bytes(const pack3d_index* index, const pack3d_attn* attn, int for_backward);

/* Forward ("Geometry Matters in Packed 3D Attention", abstract: local neighbourhood
 * attention is kept exact, only distant context is compressed into contiguous 3D block
 * summaries, every query-key and query-summary logit carries axial RoPE on the true grid
 * coordinates, and the rotation is applied before a block is summarized; local and summary
 * logits share one softmax).  Writes out [T, H, D] (attn->dtype) and lse [B, H, Nmax] fp32:
 * lse is the natural-log log-sum-exp of the scaled local and summary logits of each query.
 * coords_dev must hold the coordinates the index was built from: the RoPE angles
 * are taken from them (relative to each volume's origin, which leaves every logit
 * unchanged).  Mismatched coordinates give unspecified values but no out-of-bounds
 * access.  Precision: fp32 inputs are computed in fp32 throughout; bf16 inputs use
 * bf16 matrix-core products with fp32 accumulation and fp32 softmax.  q, k, v, out and
 * the workspace must be 16-byte aligned (PACK3D_E_INVALID otherwise). */
pack3d_status pack3d_forward(const pack3d_index* index, const pack3d_attn* attn,
                             const void* q_dev, const void* k_dev, const void* v_dev,
                             const int32_t* coords_dev, void* out_dev, float* lse_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream);

/* Backward ("Geometry Matters in Packed 3D Attention", abstract: the operator is
 * trainable at scale) of sum(out * dout): gradients dq, dk, dv [T, H, D] (attn->dtype) with
 * respect to the unrotated q, k, v, through the RoPE and the block mean pooling (a
 * block's mean spreads 1/n_b to each of its n_b present tokens).
 * out_dev and lse_dev are the forward's outputs for the same inputs.  The workspace
 * needs pack3d_workspace_bytes(index, attn, 1) bytes; its first
 * pack3d_workspace_bytes(index, attn, 0) bytes have the forward's layout.
 * reuse_forward = 0: the rotated and pooled operands are recomputed from q, k, v.
 * reuse_forward = 1: the caller guarantees that those first bytes still hold what
 * pack3d_forward wrote for the same index, attn, q, k, v and coords (same workspace
 * pointer, untouched since), and the recomputation is skipped; results are then
 * bitwise equal to reuse_forward = 0.  A broken guarantee gives wrong gradients but
 * no out-of-bounds access.  Other values: PACK3D_E_INVALID.  q, k, v, out, dout, dq, dk,
 * dv and the workspace must be 16-byte aligned (PACK3D_E_INVALID otherwise). */
pack3d_status pack3d_backward(const pack3d_index* index, const pack3d_attn* attn,
                              const void* q_dev, const void* k_dev, const void* v_dev,
                              const int32_t* coords_dev, const void* out_dev,
                              const float* lse_dev, const void* dout_dev, void* dq_dev,
                              void* dk_dev, void* dv_dev, void* workspace_dev,
                              size_t workspace_bytes, int32_t reuse_forward, void* stream);

/* Fused-projection layout ("Geometry Matters in Packed 3D Attention", abstract: the operator
 * is trained at scale inside a transformer, whose QKV projection emits one [T, 3 * H * D]
 * matrix).  Same operator as pack3d_forward / pack3d_backward, but q, k and v are read from
 * one contiguous qkv buffer [T, 3, H, D] (attn->dtype; q = qkv[:, 0], k = qkv[:, 1],
 * v = qkv[:, 2]) and the backward writes the gradients into one dqkv buffer of that layout,
 * so no split or concatenation copy is needed around the projection.  out, lse, dout and the
 * workspace are as in pack3d_forward / pack3d_backward; results are bitwise equal to them.
 * heads * head_dim * element size must be a multiple of 16 bytes (PACK3D_E_UNSUPPORTED
 * otherwise); qkv and dqkv must be 16-byte aligned. */
pack3d_status pack3d_forward_qkv(const pack3d_index* index, const pack3d_attn* attn, const void* qkv_dev,
                                 const int32_t* coords_dev, void* out_dev, float* lse_dev,
                                 void* workspace_dev, size_t workspace_bytes, void* stream);
pack3d_status pack3d_backward_qkv(const pack3d_index* index, const pack3d_attn* attn, const void* qkv_dev,
                                  const int32_t* coords_dev, const void* out_dev, const float* lse_dev,
                                  const void* dout_dev, void* dqkv_dev, void* workspace_dev,
                                  size_t workspace_bytes, int32_t reuse_forward, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pack3d_forward with the workspace
 * taken from a fixed device buffer the library holds, PACK3D_NOALLOC_MAX_BYTES (128 MiB)
 * on every GPU it runs on, kept until the process ends.  Arguments, results and errors
 * are those of pack3d_forward (bitwise equal results); there is no workspace argument.
 * The call allocates nothing: no hipMalloc / hipFree, no host allocation, no HIP events
 * (kernel timing records nothing during it).  Its first call on a device, with that device
 * current, looks up the buffer's address there (hipGetSymbolAddress) and keeps it.
 * Returns PACK3D_E_WORKSPACE, before any launch, when the forward needs more than
 * PACK3D_NOALLOC_MAX_BYTES of workspace (pack3d_workspace_bytes(index, attn, 0)).  Every
 * call on one GPU shares that GPU's buffer: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give wrong results; calls on one stream are
 * ordered and safe.  The buffer keeps the last call's contents; nothing in it needs to
 * start at zero. */
#define PACK3D_NOALLOC_MAX_BYTES ((size_t)128 << 20)
pack3d_status pack3d_forward_noalloc(const pack3d_index* index, const pack3d_attn* attn,
                                     const void* q_dev, const void* k_dev, const void* v_dev,
                                     const int32_t* coords_dev, void* out_dev, float* lse_dev,
                                     void* stream);

/* Plumbing (no passage defines this call): where the forward leaves its intermediates
 * inside the workspace (byte offsets), for inspection by tests.  All arrays are in canonical order (block-major, raster
 * inside each block; empty slots hold zero rows), elements of attn->dtype except
 * rope_table (float2 cos, sin).  N below is nblk * |b| canonical rows per volume.
 *   rope_table [extent_table, P]     cos and sin of angle row r, pair k; P = D/6 pairs per
 *                                    axis group (axial), D/2 (packed 1D) or D/2 with the
 *                                    single row 0 (no rotation)
 *   qrot, krot, vrow [B, H, N, Dp]   rotated Q and K, and V, rows zero-padded to Dp
 *   kbar, vbar [B, H, nblk_pad, Dp]  block means (over present tokens) of the rotated K and
 *                                    of V (zero rows for empty and padding blocks); written
 *                                    only with with_summaries = 1 (the windowed-only
 *                                    attention reads no block means)
 * Axial rotation angles use coordinates relative to each volume's origin (rows =
 * extents); packed 1D angles use the local packed position (rows = Nmax). */
typedef struct pack3d_views {
  size_t rope_table, qrot, krot, vrow, kbar, vbar;
  int32_t head_dim_padded, nblk_padded, extent_table;
} pack3d_views;
pack3d_status pack3d_workspace_views(const pack3d_index* index, const pack3d_attn* attn,
                                     pack3d_views* out);

/* Kernel timing, for measurement (plumbing; no passage defines these calls).  While enabled, every kernel launch made by
 * pack3d_forward / pack3d_backward is bracketed by two HIP events recorded on the
 * caller's stream (the stream the kernel runs on).  pack3d_profile_read waits for
 * the recorded events, folds them into per-kernel totals and returns, for up to
 * max_kernels kernels, the kernel name (NUL-separated in names, at most 47 bytes
 * each), the number of launches and the summed milliseconds since the last reset;
 * the return value is the number of kernels written, or -1 on a HIP error.
 * Process-wide; enable before the calls to time, from one host thread. */
pack3d_status pack3d_profile_enable(int32_t enable);
int32_t pack3d_profile_read(char* names, size_t names_bytes, int32_t* launches, double* total_ms,
                            int32_t max_kernels);
void pack3d_profile_reset(void);

/* Plumbing (no passage defines these calls): thread-local message describing the last
 * error (empty string if none), and the ABI version. */
const char* pack3d_last_error(void);

/* major * 100 + minor */
int32_t pack3d_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PACK3D_H */
