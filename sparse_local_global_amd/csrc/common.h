// Internal helpers shared by the PACK3D HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pack3d.h"

namespace pack3d {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Error reporting (thread-local message, see pack3d_last_error).
pack3d_status set_error(pack3d_status st, const char* fmt, ...);
pack3d_status check_launch(const char* what);

// Kernel timing (pack3d_profile_*): bracket a launch with events on stream s.
struct ProfileScope {
  ProfileScope(const char* name, hipStream_t s);
  ~ProfileScope();
  int slot;
  hipStream_t stream;
};

// While one is alive on a thread, ProfileScope records nothing on that thread (no events
// are created and no host memory is taken), whatever pack3d_profile_enable says.
struct ProfileOff {
  ProfileOff();
  ~ProfileOff();
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Geometry record per volume, stored in device memory as int32[G_FIELDS]: origin,
// extent, status, offending token, tokens of the volume, blocks of the volume.
enum GeomField { G_OZ = 0, G_OY, G_OX, G_EZ, G_EY, G_EX, G_STATUS, G_TOKEN, G_NTOK, G_NBLK, G_FIELDS };
// Values of G_STATUS.
enum GeomStatus { GS_OK = 0, GS_GRID = 1, GS_DIVISIBLE = 2, GS_DUPLICATE = 3, GS_EMPTY = 4, GS_BLOCKS = 5 };

}  // namespace pack3d

// Host-side index handle (opaque to callers).  Canonical arrays hold nblk * bvol rows per
// volume (nblk = the largest block count of the batch); a slot with no token is empty.
struct pack3d_index {
  int32_t batch, tokens, nblk, bvol, slots, radius;  // tokens: largest volume
  int32_t ragged, holes;   // holes: some canonical slot is empty (masking needed)
  int64_t total;           // tokens of the whole batch
  int32_t block[3];
  int32_t extent_max[3];
  int32_t* geom;         // device [B, G_FIELDS]
  int32_t* voff;         // device [B + 1] token offset of each volume
  int32_t* token_block;  // device [T]
  int32_t* canon;        // device [T]
  int32_t* perm;         // device [B, nblk * bvol], -1 = empty slot
  int32_t* nbr;          // device [B, nblk, slots]
  int32_t* count;        // device [B, nblk] tokens present per block
  uint32_t* occ;         // device [B, occ_words] bit per canonical slot: token present
  uint32_t* emask;       // device [B, nblkp / 32] bit per block: empty (no summary)
  int32_t occ_words;
  int32_t* host_geom;    // host copy [B, G_FIELDS]
};
