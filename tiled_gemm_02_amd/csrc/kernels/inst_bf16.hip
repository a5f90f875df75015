// inst_bf16.hip -- kernel instances and launchers for bf16 storage.
#include <algorithm>
#define TG_TRAIT BF16
#define TG_NAME bf16
// macro tiles of the LDS-DMA kernels
#define TG_TILE_LIST TG_TILE(256, 256) TG_TILE(256, 128) TG_TILE(128, 128) TG_TILE(128, 64) TG_TILE(64, 64)
// tiles of the four-wave kernel also built with K groups per workgroup (tile,
// groups; four waves per group)
#define TG_KG_TILE_LIST TG_TILE_KG(128, 128, 2) TG_TILE_KG(64, 64, 4)
// 16-bit vector loads run on the LDS-DMA kernels only: the register-staged
// kernel keeps its element-wise 64 x 64 form for operands off the 16-byte grid
#define TG_REG_TILE_LIST
// of those, the ones also built with K groups per workgroup (tile, groups)
#define TG_REG_KG_TILE_LIST
#define TG_HAS_MFMA2 1
#define TG_HAS_SKINNY 1
#include "instances.inc"
