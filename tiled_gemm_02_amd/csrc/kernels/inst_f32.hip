// inst_f32.hip -- kernel instances and launchers for f32 storage.
#include <algorithm>
#define TG_TRAIT F32
#define TG_NAME f32
#define TG_REG_TILE_LIST TG_TILE(128, 128) TG_TILE(64, 64)
// of those, the ones also built with K groups per workgroup (tile, groups)
#define TG_REG_KG_TILE_LIST TG_TILE_KG(128, 128, 2) TG_TILE_KG(64, 64, 4) TG_TILE_KG(32, 32, 4)
#define TG_HAS_MFMA2 0
#define TG_HAS_PP_NT 1     // the ping-pong kernel, K-contiguous operands
#define TG_HAS_SKINNY 0
#include "instances.inc"
