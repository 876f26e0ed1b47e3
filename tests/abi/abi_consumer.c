/* A plain C consumer of include/pack3d.h, built with gcc by tests/test_abi_cpu.py.
 *
 * It prints, one "name value" pair per line, the size and field offsets of every struct
 * the header declares and the value of every enumerator, as the C compiler lays them out;
 * the test compares them with the ctypes declarations of the Python binding.  Linked
 * against libpack3d.so (argument "call"), it also calls the entry points that need no
 * GPU: the version, the index size query and argument errors of the index builder, which
 * are refused before any HIP call. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "pack3d.h"

#define SIZE(T) printf("sizeof.%s %zu\n", #T, sizeof(T))
#define OFF(T, f) printf("offsetof.%s.%s %zu\n", #T, #f, offsetof(T, f))
#define ENUM(e) printf("enum.%s %d\n", #e, (int)(e))

static void layout(void) {
  SIZE(pack3d_packing);
  OFF(pack3d_packing, batch); OFF(pack3d_packing, tokens_per_volume); OFF(pack3d_packing, order_hint);
  OFF(pack3d_packing, ragged); OFF(pack3d_packing, volume_offsets); OFF(pack3d_packing, max_blocks);
  SIZE(pack3d_attn);
  OFF(pack3d_attn, dtype); OFF(pack3d_attn, heads); OFF(pack3d_attn, head_dim); OFF(pack3d_attn, rope_base);
  OFF(pack3d_attn, softmax_scale); OFF(pack3d_attn, with_summaries); OFF(pack3d_attn, position_mode);
  SIZE(pack3d_tables);
  OFF(pack3d_tables, token_block); OFF(pack3d_tables, canon); OFF(pack3d_tables, perm); OFF(pack3d_tables, nbr);
  OFF(pack3d_tables, geom); OFF(pack3d_tables, batch); OFF(pack3d_tables, tokens); OFF(pack3d_tables, nblk);
  OFF(pack3d_tables, block_tokens); OFF(pack3d_tables, slots); OFF(pack3d_tables, radius);
  OFF(pack3d_tables, block_shape); OFF(pack3d_tables, extent_max); OFF(pack3d_tables, block_count);
  OFF(pack3d_tables, volume_offsets); OFF(pack3d_tables, total_tokens); OFF(pack3d_tables, ragged);
  OFF(pack3d_tables, holes);
  SIZE(pack3d_views);
  OFF(pack3d_views, rope_table); OFF(pack3d_views, qrot); OFF(pack3d_views, krot); OFF(pack3d_views, vrow);
  OFF(pack3d_views, kbar); OFF(pack3d_views, vbar); OFF(pack3d_views, head_dim_padded);
  OFF(pack3d_views, nblk_padded); OFF(pack3d_views, extent_table);
  ENUM(PACK3D_OK); ENUM(PACK3D_E_INVALID); ENUM(PACK3D_E_COORDS); ENUM(PACK3D_E_UNSUPPORTED);
  ENUM(PACK3D_E_WORKSPACE); ENUM(PACK3D_E_HIP);
  ENUM(PACK3D_F32); ENUM(PACK3D_BF16);
  ENUM(PACK3D_ORDER_ANY); ENUM(PACK3D_ORDER_RASTER); ENUM(PACK3D_ORDER_MORTON);
  ENUM(PACK3D_ORDER_BLOCK_CONTIGUOUS); ENUM(PACK3D_ORDER_RANDOM);
  ENUM(PACK3D_POS_AXIAL); ENUM(PACK3D_POS_PACKED_1D); ENUM(PACK3D_POS_NONE);
}

#ifdef PACK3D_LINKED
static int calls(void) {
  printf("call.version %d\n", (int)pack3d_version());
  pack3d_packing pk;
  memset(&pk, 0, sizeof(pk));
  pk.batch = 2;
  pk.tokens_per_volume = 65536;
  const int32_t block[3] = {4, 4, 4};
  printf("call.index_bytes %zu\n", pack3d_index_bytes(&pk, block, 1));
  pk.tokens_per_volume = 100; /* not a whole number of 64-token blocks */
  printf("call.index_bytes_bad %zu\n", pack3d_index_bytes(&pk, block, 1));
  pack3d_index* ix = NULL;
  pk.tokens_per_volume = 65536;
  /* a null coordinate pointer is refused before any HIP call */
  pack3d_status st = pack3d_build_index(NULL, &pk, block, 1, NULL, 0, NULL, &ix);
  printf("call.build_index_null %d\n", (int)st);
  printf("call.build_index_null_message %s\n", strlen(pack3d_last_error()) > 0 ? "set" : "empty");
  printf("call.handle_null %d\n", ix == NULL);
  return 0;
}
#endif

int main(int argc, char** argv) {
  layout();
#ifdef PACK3D_LINKED
  if (argc > 1 && strcmp(argv[1], "call") == 0) return calls();
#else
  (void)argc;
  (void)argv;
#endif
  return 0;
}
