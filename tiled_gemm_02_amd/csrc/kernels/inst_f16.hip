// inst_f16.hip -- kernel instances and launchers for f16 storage.
#include <algorithm>
#define TG_TRAIT F16
#define TG_NAME f16
#define TG_TILE_LIST TG_TILE(256, 256) TG_TILE(256, 128) TG_TILE(128, 128) TG_TILE(128, 64) TG_TILE(64, 64)
#define TG_HAS_MFMA2 1
#define TG_HAS_SKINNY 1
#include "instances.inc"
